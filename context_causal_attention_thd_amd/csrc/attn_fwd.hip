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
// of one (document piece, head); each wave owns 32 query rows as two 16-row
// blocks. Keys are walked from the document start in 64-key tiles,
// double-buffered in LDS (row-major K and V). Everything is computed in the
// transposed form
//   S^T = K Q^T  and  O^T = V^T P^T
// with v_mfma_f32_16x16x32_bf16: lane l owns query column l%16 of each block
// and keys 4*(l/16) + i of every 16-key block. Each K fragment (one 16-byte
// LDS read) and each V^T fragment (two transposing LDS reads) feeds the MFMAs
// of both query blocks, which halves the LDS bytes per MFMA against 16-row
// waves; the transposing reads run at half the LDS rate of 16-byte reads, so
// this is what keeps the kernel MFMA-bound. P feeds the second product with no
// data movement.
//
// The next tile's K/V rows are fetched with buffer loads whose descriptor ends
// at the last attended key: rows past it read as zero with no branch, so the
// loads are unconditional, stay in flight during the current tile's MFMAs and
// are only waited for when they are written to LDS. Padding never enters a
// product.
//
// Online softmax in the log2 domain with lazy rescaling: the running max of a
// query only moves when a tile's scores exceed it by more than kRescaleLog2,
// so probabilities stay below 2^kRescaleLog2 (exact in fp32, representable in
// bf16) and the accumulator rescale, with its cross-lane max, runs only on the
// rare tiles where some lane of the wave crosses that bound (a wave vote). The
// row sum is kept per lane and reduced across the four 16-lane groups once, at
// the end. Only tiles on the causal diagonal apply a per-element mask.
#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.f;
static_assert(kWaves * kRowsPerWave == kFwdBM, "query tile = waves x rows per wave");

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
  constexpr int CPR = D / 8;   // 16-byte chunks per row
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

  // Query rows of this lane: block qb holds tile row w*32 + qb*16 + l16.
  int my_g[2];
  bool in_tile[2];
  int64_t m_row[2];
  bf16x8 qf[2][KS];  // B operand of S^T: query l16, head dims kk*32 + G*8 .. +7
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int r = w * kRowsPerWave + qb * 16 + l16;
    in_tile[qb] = r < t.n;
    const int g = t.g0 + r;
    const bool valid = in_tile[qb] && g < t.e;
    m_row[qb] = (int64_t)t.m0 + r;
    my_g[qb] = valid ? g : -1;  // key j is allowed iff j <= my_g
    const bf16* qp = q + m_row[qb] * rs + head_off + G * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qf[qb][kk] = valid ? load_bf16x8(qp + kk * 32) : zero_bf16x8();
  }

  f32x4 oacc[2][NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[qb][nb][i] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_part[2] = {0.f, 0.f};  // this lane's share of the row sum

  const int row0 = w * kRowsPerWave;
  const bool wave_has_rows = (row0 < t.n) && (t.g0 + row0 < t.e);
  const int wrow_last = min(row0 + kRowsPerWave - 1, t.n - 1);
  const int wave_kmax = wave_uniform(wave_has_rows ? min(t.g0 + wrow_last, t.e - 1) : -1);
  const int wave_gmin = wave_uniform(t.g0 + row0);
  const bool wave_all_valid = wave_uniform((row0 + kRowsPerWave - 1 < t.n) &&
                                           (t.g0 + row0 + kRowsPerWave - 1 < t.e)) != 0;

  // Per-thread staging slots: chunk c = threadIdx + j*kThreads is row c/CPR,
  // 16-byte column c%CPR of the tile.
  uint32_t goff[CH];
  int soff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = threadIdx.x + j * kThreads;
    const int kr = c / CPR, dc = c - kr * CPR;
    goff[j] = (uint32_t)(kr * rs * 2 + dc * 16);
    soff[j] = kr * P + dc * 8;
  }
  u32x4 kreg[CH], vreg[CH];
  auto load_tile = [&](int k0) {
    // Descriptor from key k0 to the last attended key: later rows read 0.
    const int64_t base = (int64_t)k0 * rs + head_off;
    const uint32_t bytes = (uint32_t)((int64_t)(t.kend - k0) * rs * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + base, bytes);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      kreg[j] = buffer_load16(rk, goff[j]);
      vreg[j] = buffer_load16(rv, goff[j]);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      *reinterpret_cast<u32x4*>(&sm.k[buf][soff[j]]) = kreg[j];
      *reinterpret_cast<u32x4*>(&sm.v[buf][soff[j]]) = vreg[j];
    }
  };

  const int ntiles = t.kend > t.a ? (t.kend - t.a + BN - 1) / BN : 0;
  if (ntiles > 0) {
    load_tile(t.a);
    store_tile(0);
  }
  // The Q fragments (and the first tile) have landed before the loop, so the
  // loop's MFMAs never wait on the prefetch loads issued inside it.
  wait_vmem();
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int k0 = t.a + it * BN;
    const int cur = it & 1;
    const bool has_next = it + 1 < ntiles;
    if (has_next) load_tile(k0 + BN);  // in flight during this tile's compute

    if (k0 <= wave_kmax) {
      // S^T (keys x queries): one 16x16 accumulator per (query block, key block).
      f32x4 s[2][KB];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[qb][kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 a = load_bf16x8(&sm.k[cur][(kb * 16 + l16) * P + kk * 32 + G * 8]);
          s[0][kb] = mfma16(a, qf[0][kk], s[0][kb]);
          s[1][kb] = mfma16(a, qf[1][kk], s[1][kb]);
        }

      // Causal / padding mask, only where some key may exceed some row's g.
      if (!wave_all_valid || k0 + BN - 1 > wave_gmin) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + kb * 16 + G * 4 + i;
              if (key > my_g[qb]) s[qb][kb][i] = -INFINITY;
            }
      }

      // Lazy rescale: does any score of this lane exceed its running max by
      // more than the bound?
      float lm[2];
      bool need = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[qb][kb][i]);
        lm[qb] = mx * scale_log2;
        need |= lm[qb] > m_run[qb] + kRescaleLog2;
      }
      if (__any(need)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float rm = group_max4(lm[qb]);  // the row's tile max (uniform per query)
          const float m_new = rm > m_run[qb] + kRescaleLog2 ? rm : m_run[qb];
          const float alpha = m_new == m_run[qb] ? 1.f : fast_exp2(m_run[qb] - m_new);
          m_run[qb] = m_new;
          l_part[qb] *= alpha;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[qb][nb][i] *= alpha;
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(fmaf(s[qb][kb][i], scale_log2, -m_use));
            s[qb][kb][i] = p;
            ps += p;
          }
        l_part[qb] += ps;
      }

      // O^T += V^T P^T. k-step ks covers key blocks 2ks, 2ks+1: slot j of this
      // lane is key (2ks + j/4)*16 + 4*G + j%4 -- accumulator entries of
      // s[.][2ks], s[.][2ks+1]. The V^T operand (lane = head dim, slots = those
      // keys) is two transposing reads of the row-major V tile, shared by both
      // query blocks.
#pragma unroll
      for (int ks = 0; ks < KB / 2; ++ks) {
        const bf16x8 pb0 = pack8(s[0][2 * ks], s[0][2 * ks + 1]);
        const bf16x8 pb1 = pack8(s[1][2 * ks], s[1][2 * ks + 1]);
        const int o1 = (2 * ks * 16 + G * 4 + (l16 >> 2)) * P + 4 * (l16 & 3);
        const int o2 = o1 + 16 * P;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 a = concat4(lds_read_tr4(&sm.v[cur][o1 + nb * 16]),
                                   lds_read_tr4(&sm.v[cur][o2 + nb * 16]));
          oacc[0][nb] = mfma16(a, pb0, oacc[0][nb]);
          oacc[1][nb] = mfma16(a, pb1, oacc[1][nb]);
        }
      }
    }

    if (has_next) store_tile(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = group_sum4(l_part[qb]);
    if (!in_tile[qb]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    bf16* op = o + m_row[qb] * rs + head_off;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // accumulator rows (head dims) nb*16 + 4*G + 0..3 of query l16
      bf16x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = (bf16)(oacc[qb][nb][j] * inv);
      store_bf16x4(op + nb * 16 + G * 4, out);
    }
    if (G == 0) {
      lse[(int64_t)h * n_local + m_row[qb]] =
          (my_g[qb] >= 0 && l > 0.f) ? (m_run[qb] + __log2f(l)) * kLn2 : -INFINITY;
    }
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
