// Backward, key side: this rank's partial dK/dV over the full K/V ("[PyTorch]
// Add no-load-balance THD all-gather CP", sequence diagram: the dK/dV partials
// are unrestored for the reduce-scatter). dQ is computed by the query-major
// kernel in attn_bwd_dq.hip, so this kernel needs no atomics and every key row
// it owns is written by exactly one workgroup. Padding never enters a product:
// query rows that are not real tokens are not listed, key rows past the tile
// end are zeroed, and masked probabilities are selected to 0 (NaN-safe).
//
// gfx950 design: a workgroup of 4 waves owns 128 consecutive keys of one
// document (32 per wave, K and V fragments in registers) and walks the local
// query rows that attend them in blocks of 64. Query blocks (Q, dO, LSE,
// delta) are double-buffered in LDS and the next block's global loads are in
// flight while the current one is computed; one barrier per block. Per block
// each wave computes with v_mfma_f32_32x32x16_bf16
//   S = Q K^T, dP = dO V^T          (A = Q / dO rows from LDS, B = K / V regs)
//   P = exp(S - LSE), dS = P (dP - delta)
//   dV += P^T dO, dK += dS^T Q       (accumulators stay in registers)
// P and dS come out of the first products already in the A-operand layout of
// the last two; their B operands (dO and Q, sliced by column) are transposing
// LDS reads of the row-major tiles.
#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 64;  // query rows per block (two 32-query halves)
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BwdSmem {
  static constexpr int P = D + 16;     // Q / dO row pitch (bf16)
  bf16 q[2][kBM * P];
  bf16 dO[2][kBM * P];
  float lse2[2][kBM];
  float dlt[2][kBM];
  int32_t gq[2][kBM];
};

template <int D>
__global__ void __launch_bounds__(kThreads, 1)
attn_bwd_dkdv_kernel(const BwdTile* __restrict__ tiles, int32_t H, const bf16* __restrict__ q,
                     const bf16* __restrict__ k, const bf16* __restrict__ v,
                     const bf16* __restrict__ d_o, const float* __restrict__ lse,
                     const float* __restrict__ delta, float* __restrict__ dk,
                     float* __restrict__ dv, int64_t n_local, float scale, float scale_log2,
                     int32_t accumulate) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int CH = kBM * CPR / kThreads;    // chunks per thread per block and tensor
  typedef BwdSmem<D> S;
  constexpr int P = S::P;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  S& sm = *reinterpret_cast<S*>(smem_raw);

  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const BwdTile t = tiles[tile_id];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int sl = lane & 15;
  const int g16 = lane >> 4;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = (int64_t)h * D;

  // This lane's key (column of S and dP; row of the dK/dV A operands).
  const int my_key = t.k0 + w * 32 + li;
  const bool key_ok = my_key < t.k1;
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const int64_t off = (int64_t)my_key * rs + head_off + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      kf[kk] = key_ok ? load_bf16x8(k + off + kk * 16) : zero_bf16x8();
      vf[kk] = key_ok ? load_bf16x8(v + off + kk * 16) : zero_bf16x8();
    }
  }
  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[db][i] = 0.f;
      dva[db][i] = 0.f;
    }

  // Query-block staging: chunk c = threadIdx.x + j*kThreads of the block.
  bf16x8 qreg[CH], dreg[CH];
  float lreg = 0.f, dlreg = 0.f;
  int greg = -1;
  auto load_block = [&](int mb) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int rr = c / CPR, dc = c - rr * CPR;
      const int m = mb + rr;
      const int64_t off = (int64_t)m * rs + head_off + dc * 8;
      qreg[j] = m < t.m_hi ? load_bf16x8(q + off) : zero_bf16x8();
      dreg[j] = m < t.m_hi ? load_bf16x8(d_o + off) : zero_bf16x8();
    }
    if (threadIdx.x < kBM) {
      const int m = mb + threadIdx.x;
      const bool ok = m < t.m_hi;
      lreg = ok ? lse[(int64_t)h * n_local + m] * kLog2e : 0.f;
      dlreg = ok ? delta[(int64_t)h * n_local + m] : 0.f;
      greg = ok ? m + (m < t.m_split ? t.dg_a : t.dg_b) : -1;
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = threadIdx.x + j * kThreads;
      const int rr = c / CPR, dc = c - rr * CPR;
      store_bf16x8(&sm.q[buf][rr * P + dc * 8], qreg[j]);
      store_bf16x8(&sm.dO[buf][rr * P + dc * 8], dreg[j]);
    }
    if (threadIdx.x < kBM) {
      sm.lse2[buf][threadIdx.x] = lreg;
      sm.dlt[buf][threadIdx.x] = dlreg;
      sm.gq[buf][threadIdx.x] = greg;
    }
  };

  const int nblocks = (t.m_hi - t.m_lo + kBM - 1) / kBM;
  load_block(t.m_lo);
  store_block(0);
  __syncthreads();

  for (int it = 0; it < nblocks; ++it) {
    const int mb = t.m_lo + it * kBM;
    const int cur = it & 1;
    const bool has_next = it + 1 < nblocks;
    if (has_next) load_block(mb + kBM);  // in flight during this block's compute

    // S and dP for the two 32-query halves (rows = queries, column = my_key).
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[qb][i] = 0.f;
        dp[qb][i] = 0.f;
      }
      const bf16* qa = &sm.q[cur][(qb * 32 + li) * P + hh * 8];
      const bf16* da = &sm.dO[cur][(qb * 32 + li) * P + hh * 8];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s[qb] = mfma32(load_bf16x8(qa + kk * 16), kf[kk], s[qb]);
        dp[qb] = mfma32(load_bf16x8(da + kk * 16), vf[kk], dp[qb]);
      }
    }
    // Element i of s[qb]: query row qb*32 + 8*(i/4) + 4*hh + i%4, key my_key.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int qr0 = qb * 32 + i4 * 8 + hh * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[cur][qr0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[cur][qr0]);
        const i32x4 g4 = *reinterpret_cast<const i32x4*>(&sm.gq[cur][qr0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i4 * 4 + j;
          // bitwise & keeps the LDS read unconditional (no divergent branch)
          const bool ok = key_ok & (my_key <= g4[j]);
          const float p = ok ? fast_exp2(fmaf(s[qb][i], scale_log2, -l4[j])) : 0.f;
          const float dsv = ok ? p * (dp[qb][i] - d4[j]) : 0.f;
          s[qb][i] = p;
          dp[qb][i] = dsv;
        }
      }
    // dV += P^T dO and dK += dS^T Q. k-step (qb, u) covers query rows
    // qb*32 + 16u + (j/4)*8 + hh*4 + j%4 for slot j: accumulator entries
    // u*8..u*8+7 of s[qb] / dp[qb]. The B operands (lane = head dim, slots =
    // those rows) are two transposing reads each of the row-major dO and Q.
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pa = to_bf16x8(s[qb], u * 8);
        const bf16x8 dsa = to_bf16x8(dp[qb], u * 8);
        const int roff = (qb * 32 + 16 * u + hh * 4 + (sl >> 2)) * P + 16 * (g16 & 1) + 4 * (sl & 3);
        const bf16* dob = &sm.dO[cur][roff];
        const bf16* qbp = &sm.q[cur][roff];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 bdo = concat4(lds_read_tr4(dob + db * 32), lds_read_tr4(dob + db * 32 + 8 * P));
          dva[db] = mfma32(pa, bdo, dva[db]);
          const bf16x8 bq = concat4(lds_read_tr4(qbp + db * 32), lds_read_tr4(qbp + db * 32 + 8 * P));
          dka[db] = mfma32(dsa, bq, dka[db]);
        }
      }
    if (has_next) store_block(cur ^ 1);
    __syncthreads();
  }

  // dK (scaled) and dV rows of this wave's keys; lane li holds head dim db*32 + li.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = t.k0 + w * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
      if (key < t.k1) {
        const int64_t off = (int64_t)key * rs + head_off + db * 32 + li;
        const float kval = dka[db][i] * scale;
        const float vval = dva[db][i];
        if (accumulate) {
          dk[off] += kval;
          dv[off] += vval;
        } else {
          dk[off] = kval;
          dv[off] = vval;
        }
      }
    }
}

template <int D>
hipError_t launch_bwd_d(const BwdTile* tiles, int32_t n_tiles, int32_t H, const void* q,
                        const void* k, const void* v, const void* d_o, const float* lse,
                        const float* delta, float* dk, float* dv, int64_t n_local,
                        float scale, int32_t accumulate, hipStream_t stream) {
  const int64_t blocks = (int64_t)n_tiles * H;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const size_t smem = sizeof(BwdSmem<D>);
  // The dynamic-LDS limit is a per-device function attribute: set it once per device.
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), smem,
                     stream, tiles, H, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(d_o), lse, delta, dk,
                     dv, n_local, scale, scale * kLog2e, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_dkdv(const BwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                                const void* q, const void* k, const void* v, const void* d_o,
                                const float* lse, const float* delta, float* dk, float* dv,
                                int64_t n_local, float scale, int32_t accumulate,
                                hipStream_t stream) {
  if (D == 128)
    return launch_bwd_d<128>(tiles, n_tiles, H, q, k, v, d_o, lse, delta, dk, dv, n_local,
                             scale, accumulate, stream);
  if (D == 64)
    return launch_bwd_d<64>(tiles, n_tiles, H, q, k, v, d_o, lse, delta, dk, dv, n_local,
                            scale, accumulate, stream);
  return hipErrorInvalidValue;
}

}  // namespace thdcp
