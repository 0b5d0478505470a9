/*
 * CPU oracle for the gated delta rule recurrence with dynamic state fake-quantization.
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the bench's CPU
 * baseline; never by the library.  All tensors are host float64 arrays, row-major:
 *   q, k [B][T][H][dk]; v, o, dout [B][T][H][dv]; g [B][T][H] (scalar gate) or
 *   [B][T][H][dk] (per key channel); beta [B][T][H]; S0, ST, dS0, dST [B][H][dk][dv];
 *   ckpts [B][H][ceil(T/ckpt_interval)][dk][dv] (state entering tokens 0, n, 2n, ...).
 */
#ifndef LA_ORACLE_H
#define LA_ORACLE_H
#include <stdint.h>

enum { ORACLE_GATE_SCALAR = 0, ORACLE_GATE_KEY = 1 };
enum { ORACLE_QDQ_NONE = 0, ORACLE_QDQ_INT8 = 1, ORACLE_QDQ_E4M3 = 2 };

typedef struct {
    int B, T, H, dk, dv;
    int gate;          /* ORACLE_GATE_* */
    int qdq;           /* ORACLE_QDQ_* */
    int group;         /* INT8 group width / E4M3 tile width along the value axis */
    int hadamard;      /* 1: normalized Walsh-Hadamard rotation of the key axis around INT8 */
    int qdq_interval;  /* 1: every token; n: after tokens n, 2n, ... and after the last */
    int ckpt_interval; /* 0: no checkpoints */
    int replay;        /* 1: replay windows of qdq_interval tokens (BF16 key/update entries
                          between rounding points); 0: off */
} oracle_cfg;

int oracle_num_threads(void);
void oracle_set_num_threads(int n);
double oracle_e4m3_value(int code);
int oracle_e4m3_code(double y);
void oracle_hadamard(int dk, int dv, const double* X, double* Y);
int oracle_qdq(int qdq, int group, int hadamard, int dk, int dv, const double* X, double* Xhat,
               int32_t* codes, float* scales, float* ypre);
int oracle_fwd(const oracle_cfg* c, const double* q, const double* k, const double* v,
               const double* g, const double* beta, const double* S0, double* o, double* ST,
               double* ckpts);
/* oracle_fwd with two optional arrays [B][T][H][dv]: dhat_in, in replay mode, gives the BF16
 * update entry to use at each token that is not a rounding point (a NaN entry: encode the
 * oracle's own delta); delta_out receives every token's delta (float64). */
int oracle_fwd_ex(const oracle_cfg* c, const double* q, const double* k, const double* v,
                  const double* g, const double* beta, const double* S0, double* o, double* ST,
                  double* ckpts, const double* dhat_in, double* delta_out);
double oracle_bf16(double x);
int oracle_bwd(const oracle_cfg* c, const double* q, const double* k, const double* v,
               const double* g, const double* beta, const double* S0, const double* states,
               const double* dout, const double* dST, double* dq, double* dk, double* dv,
               double* dg, double* dbeta, double* dS0);
#endif
