// Forward attention of one CP rank's local queries against the full K/V,
// masked by document boundaries and global causal position.
//
// Follows "[PyTorch] Add no-load-balance THD all-gather CP" ("Why": the rank's
// attention steps over the gathered K/V; "Scope and constraints": causal,
// window_size = (-1, 0)) and "[PyTorch] Extend no-load-balance CP to the a2a
// comm type" (body: the mask is the cp_size = 1 mask). Both DUAL_CHUNK_SWAP
// chunks of a document are separate query tiles of this one launch.
//
// gfx950 design: a workgroup of 8 waves owns up to 128 consecutive query rows
// of one (document piece, head); each wave owns 16 query rows. Keys are walked
// from the document start in 64-key tiles, double-buffered in LDS (row-major
// K and V); the next tile's global loads are issued before the current tile's
// MFMAs so their latency hides behind compute, and one barrier per tile
// suffices. Everything is computed in the transposed form
//   S^T = K Q^T  and  O^T = V^T P^T
// with v_mfma_f32_16x16x32_bf16: lane l owns query column l%16 and keys
// 4*(l/16) + i of each 16-key block, so the online-softmax max/sum need two
// exchanges across the four 16-lane groups and the rescale is lane-local; P
// feeds the second product with no data movement. V^T operands come from the
// row-major V tile through the transposing LDS read. 16-query waves keep the
// state near 100 registers, so up to four waves share a SIMD. Only tiles on
// the causal diagonal apply a per-element mask; key rows past the last
// attended key are zeroed when staged, so padding never enters a product.
#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct FwdSmem {
  // Row pitch (bf16) = D + 16: 16-byte row reads of 8 consecutive rows and
  // transposing reads of 4 consecutive rows both hit distinct banks.
  static constexpr int P = D + 16;
  bf16 k[2][kFwdBN * P];
  bf16 v[2][kFwdBN * P];
};

template <int D>
__global__ void __launch_bounds__(kThreads, 2)
attn_fwd_kernel(const FwdTile* __restrict__ tiles, int32_t H, const bf16* __restrict__ q,
                const bf16* __restrict__ k, const bf16* __restrict__ v, bf16* __restrict__ o,
                float* __restrict__ lse, int64_t n_local, float scale_log2) {
  constexpr int BN = kFwdBN;
  constexpr int KS = D / 32;   // 16x16x32 k-steps over the head dim
  constexpr int NB = D / 16;   // 16-wide blocks of the head dim
  constexpr int KB = BN / 16;  // 16-key blocks per tile
  constexpr int P = FwdSmem<D>::P;
  constexpr int CPR = D / 8;
  constexpr int CH = BN * CPR / kThreads;
  __shared__ FwdSmem<D> sm;

  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const FwdTile t = tiles[tile_id];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;  // query column of this lane (and row of A operands)
  const int G = lane >> 4;    // 16-lane group
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = (int64_t)h * D;

  const int r = w * 16 + l16;
  const bool in_tile = r < t.n;
  const int g = t.g0 + r;
  const bool valid = in_tile && g < t.e;
  const int64_t m = (int64_t)t.m0 + r;
  const int my_g = valid ? g : -1;   // key j is allowed iff j <= my_g

  // Q fragment (B operand of S^T): query l16, head dims kk*32 + G*8 .. +7
  bf16x8 qf[KS];
  {
    const bf16* qp = q + m * rs + head_off + G * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = valid ? load_bf16x8(qp + kk * 32) : zero_bf16x8();
  }

  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[nb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int wrow_last = min(w * 16 + 15, t.n - 1);
  const bool wave_has_rows = (w * 16 < t.n) && (t.g0 + w * 16 < t.e);
  const int wave_kmax = wave_uniform(wave_has_rows ? min(t.g0 + wrow_last, t.e - 1) : -1);
  const int wave_gmin = wave_uniform(t.g0 + w * 16);
  const bool wave_all_valid =
      wave_uniform((w * 16 + 15 < t.n) && (t.g0 + w * 16 + 15 < t.e)) != 0;

  bf16x8 kreg[CH], vreg[CH];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int kr = c / CPR, dc = c - kr * CPR;
      const int key = k0 + kr;
      const int64_t off = (int64_t)key * rs + head_off + dc * 8;
      kreg[j] = key < t.kend ? load_bf16x8(k + off) : zero_bf16x8();
      vreg[j] = key < t.kend ? load_bf16x8(v + off) : zero_bf16x8();
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int kr = c / CPR, dc = c - kr * CPR;
      store_bf16x8(&sm.k[buf][kr * P + dc * 8], kreg[j]);
      store_bf16x8(&sm.v[buf][kr * P + dc * 8], vreg[j]);
    }
  };

  const int ntiles = t.kend > t.a ? (t.kend - t.a + BN - 1) / BN : 0;
  if (ntiles > 0) {
    load_tile(t.a);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = t.a + it * BN;
    const int cur = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(k0 + BN);  // in flight during this tile's compute

    if (k0 <= wave_kmax) {
      // S^T (keys x queries), one 16x16 accumulator per 16-key block.
      f32x4 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          s[kb] = mfma16(load_bf16x8(&sm.k[cur][(kb * 16 + l16) * P + kk * 32 + G * 8]), qf[kk], s[kb]);

      // Causal / padding mask, only where some key may exceed some row's g.
      if (!wave_all_valid || k0 + BN - 1 > wave_gmin) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + kb * 16 + G * 4 + i;
            if (key > my_g) s[kb][i] = -INFINITY;
          }
      }

      // Online softmax in the log2 domain; the four 16-lane groups hold
      // different keys of the same queries.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(fmaf(s[kb][i], scale_log2, -m_use));
          s[kb][i] = p;
          psum += p;
        }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (!__all(alpha == 1.f)) {  // rescale only when some row's max moved
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nb][i] *= alpha;
      }

      // O^T += V^T P^T. k-step ks covers key blocks 2ks, 2ks+1: slot j of this
      // lane is key (2ks + j/4)*16 + 4*G + j%4 -- accumulator entries of
      // s[2ks], s[2ks+1]. The V^T operand (lane = head dim, slots = those
      // keys) is two transposing reads of the row-major V tile.
#pragma unroll
      for (int ks = 0; ks < KB / 2; ++ks) {
        const bf16x8 pb = pack8(s[2 * ks], s[2 * ks + 1]);
        const int o1 = (2 * ks * 16 + G * 4 + (l16 >> 2)) * P + 4 * (l16 & 3);
        const int o2 = o1 + 16 * P;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 a = concat4(lds_read_tr4(&sm.v[cur][o1 + nb * 16]), lds_read_tr4(&sm.v[cur][o2 + nb * 16]));
          oacc[nb] = mfma16(a, pb, oacc[nb]);
        }
      }
    }

    if (has_next) store_tile(cur ^ 1);
    __syncthreads();
  }

  if (!in_tile) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16* op = o + m * rs + head_off;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // accumulator rows (head dims) nb*16 + 4*G + 0..3 of query l16
    bf16x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = (bf16)(oacc[nb][j] * inv);
    store_bf16x4(op + nb * 16 + G * 4, out);
  }
  if (G == 0) {
    lse[(int64_t)h * n_local + m] =
        (valid && l_run > 0.f) ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                           const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t n_local, float scale, hipStream_t stream) {
  const int64_t blocks = (int64_t)n_tiles * H;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const float scale_log2 = scale * kLog2e;
  const bf16* qb = static_cast<const bf16*>(q);
  const bf16* kb = static_cast<const bf16*>(k);
  const bf16* vb = static_cast<const bf16*>(v);
  bf16* ob = static_cast<bf16*>(o);
  if (D == 128)
    hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       tiles, H, qb, kb, vb, ob, lse, n_local, scale_log2);
  else if (D == 64)
    hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       tiles, H, qb, kb, vb, ob, lse, n_local, scale_log2);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace thdcp
