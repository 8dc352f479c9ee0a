// Workspace layout of the chunked forward, shared by the host sizing code and
// the two chunk kernels.
//
// One block per (batch, head, chunk), blocks ordered chunk-fastest so that the
// sequential state pass streams each head's blocks contiguously.  Inside a
// block (element type Tio = the I/O dtype; KPAD = d_k rounded up to the
// matrix-core K-block, padding columns hold zeros):
//
//   qh   [64][KPAD]  Gamma_r * q_r          (chunk-level cumulative decay)
//   wwy  [64][KPAD]  W = T (Gamma * b * k)  (WY factor of the erase term)
//   ktt  [dk][64]    Ktil^T, Ktil_s = k_s * Gamma_L / Gamma_s
//   p    [64][64]    P[r][s] = sum_c q_r k_s Gamma_r/Gamma_s, s <= r (else 0)
//   gaml [dk]  fp32  Gamma_L (decay over the whole chunk)
//   uwyt [dv][64]    U^T, U = T (w * v)
//
// with T = (I + A)^{-1}, A[r][s] = sum_c b_r k_r k_s Gamma_r/Gamma_s for s < r.
// Every section starts on a 256-byte boundary.
//
// The forward recomputed for the matrix-core backward (bf16, KPAD = dk)
// writes blocks whose products contract over the token index instead: its
// qh section holds Qh^T [dk][64] and its p section P^T [64][64] (qt[c][r] =
// qh[r][c], pt[s][r] = p[r][s]), and the block continues after uwyt with
//   t    [64][64]  T
//   kn   [64][dk]  Ktil (row-major)
//   wt   [dk][64]  W^T
//   eh   [64][dk]  Eh = Gamma (b k)
#pragma once

#include <stdint.h>

namespace gdn2 {

__host__ __device__ constexpr int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct WsLayout {
    int64_t qh, wwy, ktt, p, gaml, uwyt, block;   // byte offsets and block size
};

// esize: bytes per I/O element (2 or 4); kb: K-block of the matrix core (32 or 16)
__host__ __device__ constexpr WsLayout ws_layout(int64_t dk, int64_t dv, int64_t esize, int64_t kb) {
    const int64_t kpad = (dk + kb - 1) / kb * kb;
    const int64_t qh = 0;
    const int64_t wwy = align256(qh + 64 * kpad * esize);
    const int64_t ktt = align256(wwy + 64 * kpad * esize);
    const int64_t p = align256(ktt + dk * 64 * esize);
    const int64_t gaml = align256(p + 64 * 64 * esize);
    const int64_t uwyt = align256(gaml + dk * 4);
    const int64_t block = align256(uwyt + dv * 64 * esize);
    return WsLayout{qh, wwy, ktt, p, gaml, uwyt, block};
}

// the backward's extension of a block whose forward layout ends at fwd_block
struct BwdExt {
    int64_t t, kn, wt, eh, block;
};
__host__ __device__ constexpr BwdExt bwd_ext(int64_t fwd_block, int64_t dk)
{
    return BwdExt{fwd_block, fwd_block + 64 * 64 * 2, fwd_block + 64 * 64 * 2 + 64 * dk * 2,
                  fwd_block + 64 * 64 * 2 + 2 * (64 * dk * 2), fwd_block + 64 * 64 * 2 + 3 * (64 * dk * 2)};
}

}  // namespace gdn2
