/*
 * gdn_oracle.h -- entry points of the fp64 CPU oracle (test infrastructure only).
 * Host pointers throughout.  Layouts (row-major, contiguous):
 *   q, k      [B, H, T, Dk]      v [B, H, T, Dv]
 *   beta      [B, H, T]          log_alpha [B, H, T] (GDN) or [B, H, T, Dk] (KDA)
 *   s0        [B, H, Dv, Dk]     (NULL = zeros)
 *   o         [B, H, T, Dv]      s_final [B, H, Dv, Dk]
 *   s_ckpt    [B, H, T / ckpt_every, Dv, Dk]: snapshot n = state after token (n+1)*ckpt_every
 * Decode: state [N, H, Dv, Dk] fp64 updated in place; q, k [N, H, Dk]; v [N, H, Dv];
 *   beta [N, H]; log_alpha [N, H] (GDN) or [N, H, Dk] (KDA); o [N, H, Dv].
 * Return: number of worker threads used (> 0), or -1 on a bad argument / allocation failure.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H
#include <stdint.h>

enum { ORA_F64 = 0, ORA_F32 = 1, ORA_BF16 = 2 };

int ora_forward(int64_t B, int64_t H, int64_t T, int64_t Dk, int64_t Dv, int kda, int in_dtype,
                const void* q, const void* k, const void* v, const void* beta, const void* log_alpha,
                const void* s0, int s0_dtype, double* o, double* s_final, double* s_ckpt,
                int64_t ckpt_every, int nthreads);

int ora_decode_step(int64_t N, int64_t H, int64_t Dk, int64_t Dv, int kda, int in_dtype, double* state,
                    const void* q, const void* k, const void* v, const void* beta, const void* log_alpha,
                    double* o, int nthreads);

int ora_hardware_threads(void);

#endif
