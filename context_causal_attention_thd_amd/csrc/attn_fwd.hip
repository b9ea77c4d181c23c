// Forward attention of one CP rank's local queries against the full K/V,
// masked by document boundaries and global causal position.
//
// Follows "[PyTorch] Add no-load-balance THD all-gather CP" ("Why": the rank's
// attention steps over the gathered K/V; "Scope and constraints": causal,
// window_size = (-1, 0)) and "[PyTorch] Extend no-load-balance CP to the a2a
// comm type" (body: the mask is the cp_size = 1 mask). Both DUAL_CHUNK_SWAP
// chunks of a document are separate query tiles of this one launch.
//
// gfx950 design: a workgroup of 4 waves owns up to 128 consecutive query rows
// of one (document piece, head); each wave owns 32 query rows. Keys are walked
// from the document start in 64-key tiles, double-buffered in LDS (row-major
// K and V); the next tile's global loads are issued before the current tile's
// MFMAs so their latency hides behind compute, and one barrier per tile
// suffices. Everything is computed in the transposed form
//   S^T = K Q^T  and  O^T = V^T P^T
// with v_mfma_f32_32x32x16_bf16, so every lane owns one query column of the
// accumulators: the online-softmax max/sum/rescale are lane-local apart from
// one exchange with the lane 32 away, and P feeds the second product with no
// data movement. V^T operands come from the row-major V tile through the
// transposing LDS read. Only tiles on the causal diagonal apply a per-element
// mask; key rows past the last attended key are zeroed when staged, so padding
// rows never enter a product (NaN-safe).
#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr int kWaves = 4;
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
  constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DB = D / 32;      // 32-wide blocks of the head dim
  constexpr int P = FwdSmem<D>::P;
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int CH = BN * CPR / kThreads;       // chunks per thread per tile and tensor
  __shared__ FwdSmem<D> sm;

  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const FwdTile t = tiles[tile_id];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;   // query column of this lane (and row index of A operands)
  const int hh = lane >> 5;   // which half of the wave
  const int sl = lane & 15;   // lane within its 16-lane group (transposing reads)
  const int g16 = lane >> 4;  // 16-lane group
  const int64_t rs = (int64_t)H * D;  // row stride in elements

  const int r = w * 32 + li;
  const bool in_tile = r < t.n;
  const int g = t.g0 + r;
  const bool valid = in_tile && g < t.e;
  const int64_t m = (int64_t)t.m0 + r;
  const int my_g = valid ? g : -1;   // key j is allowed iff j <= my_g (keys start at t.a >= 0)

  // Q fragment (B operand of S^T): query li, head dims kk*16 + hh*8 .. +7
  bf16x8 qf[KSTEPS];
  {
    const bf16* qp = q + m * rs + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = valid ? load_bf16x8(qp + kk * 16) : zero_bf16x8();
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Wave-level bounds: the last key any row of this wave attends, and the
  // first row's global index (every key <= it is visible to all real rows).
  const int wrow_last = min(w * 32 + 31, t.n - 1);
  const bool wave_has_rows = (w * 32 < t.n) && (t.g0 + w * 32 < t.e);
  const int wave_kmax = wave_uniform(wave_has_rows ? min(t.g0 + wrow_last, t.e - 1) : -1);
  const int wave_gmin = wave_uniform(t.g0 + w * 32);
  const bool wave_all_valid =
      wave_uniform((w * 32 + 31 < t.n) && (t.g0 + w * 32 + 31 < t.e)) != 0;

  // Staging: thread handles chunks c = threadIdx.x + j*kThreads of the tile.
  const int64_t head_off = (int64_t)h * D;
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
      // S^T (keys x queries) for the two 32-key halves of the tile.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
        const bf16* kp = &sm.k[cur][(kb * 32 + li) * P + hh * 8];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) s[kb] = mfma32(load_bf16x8(kp + kk * 16), qf[kk], s[kb]);
      }

      // Causal / padding mask, only where some key may exceed some row's g.
      if (!wave_all_valid || k0 + BN - 1 > wave_gmin) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
            if (key > my_g) s[kb][i] = -INFINITY;
          }
      }

      // Online softmax in the log2 domain (scale * log2(e) folded in).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, shfl_xor32(mx));
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[kb][i], scale_log2, -m_use));
          s[kb][i] = p;
          psum += p;
        }
      psum += shfl_xor32(psum);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (!__all(alpha == 1.f)) {  // rescale only when some row's max moved
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }

      // O^T += V^T P^T. k-step (kb, u) covers 16 keys; slot j of this lane is
      // key kb*32 + 16u + (j/4)*8 + hh*4 + j%4 -- exactly accumulator entries
      // u*8 .. u*8+7 of s[kb], so P needs no data movement. The V^T operand
      // (lane = head dim, slots = those keys) is two transposing reads of the
      // row-major V tile: rows kb*32+16u+hh*4+{0..3} and the same +8.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 pb = to_bf16x8(s[kb], u * 8);
          const bf16* vb = &sm.v[cur][(kb * 32 + 16 * u + hh * 4 + (sl >> 2)) * P +
                                      16 * (g16 & 1) + 4 * (sl & 3)];
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 a = concat4(lds_read_tr4(vb + db * 32), lds_read_tr4(vb + db * 32 + 8 * P));
            oacc[db] = mfma32(a, pb, oacc[db]);
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
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      // accumulator rows (head dims) db*32 + i4*8 + hh*4 + 0..3 of query li
      bf16x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = (bf16)(oacc[db][i4 * 4 + j] * inv);
      store_bf16x4(op + db * 32 + i4 * 8 + hh * 4, out);
    }
  if (hh == 0) {
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
