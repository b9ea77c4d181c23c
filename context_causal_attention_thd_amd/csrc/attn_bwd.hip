// Backward attention of one CP rank's share: dQ for the local rows and this
// rank's partial dK/dV over the full K/V ("[PyTorch] Add no-load-balance THD
// all-gather CP", sequence diagram: the dK/dV partials are unrestored for the
// reduce-scatter). Padding never enters a product: query rows that are not
// real tokens are not listed, key rows past the tile end are zeroed, and
// masked probabilities are selected to 0 (NaN-safe).
//
// gfx950 design: a workgroup of 4 waves owns 128 consecutive keys of one
// document (32 per wave) and walks the local query rows that attend them in
// blocks of 32. Per block, each wave computes with v_mfma_f32_32x32x16_bf16
//   S = Q K^T, dP = dO V^T   (queries x its keys; K, V fragments in registers)
//   P = exp(S - LSE), dS = P (dP - delta)
//   dV += P^T dO, dK += dS^T Q   (accumulators stay in registers)
// P and dS are already in the A-operand layout of the last two products, so
// only dO^T and Q^T are staged transposed in LDS. dS is written to LDS once
// and wave w then forms dQ for head dims [32w, 32w+32) over all 128 keys and
// adds it to global dQ with float atomics (coalesced 128-byte rows).
#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BwdSmem {
  static constexpr int QP = D + 8;         // Q / dO row-major pitch (bf16)
  static constexpr int TP = kBwdBM + 4;    // Q^T / dO^T pitch (bf16)
  static constexpr int SP = kBwdBN + 8;    // dS pitch (bf16)
  static constexpr int KTP = kBwdBN + 8;   // K^T pitch (bf16)
  bf16 q[kBwdBM * QP];
  bf16 qt[D * TP];
  bf16 dO[kBwdBM * QP];
  bf16 dOt[D * TP];
  bf16 ds[kBwdBM * SP];
  bf16 kt[D * KTP];
  float lse2[kBwdBM];
  float dlt[kBwdBM];
  int32_t gq[kBwdBM];
};

template <int D>
__global__ void __launch_bounds__(kThreads, 1)
attn_bwd_kernel(const BwdTile* __restrict__ tiles, int32_t H, const bf16* __restrict__ q,
                const bf16* __restrict__ k, const bf16* __restrict__ v,
                const bf16* __restrict__ d_o, const float* __restrict__ lse,
                const float* __restrict__ delta, float* __restrict__ dq, float* __restrict__ dk,
                float* __restrict__ dv, int64_t n_local, float scale, float scale_log2,
                int32_t accumulate) {
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  typedef BwdSmem<D> S;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  S& sm = *reinterpret_cast<S*>(smem_raw);

  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const BwdTile t = tiles[tile_id];
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int64_t rs = (int64_t)H * D;

  // This lane's key (column of S and dP; row of the dK/dV A operands).
  const int my_key = t.k0 + w * 32 + li;
  const bool key_ok = my_key < t.k1;
  const bool wave_live = t.k0 + w * 32 < t.k1;
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const int64_t off = (int64_t)my_key * rs + (int64_t)h * D + hh * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      kf[kk] = key_ok ? load_bf16x8(k + off + kk * 16) : zero_bf16x8();
      vf[kk] = key_ok ? load_bf16x8(v + off + kk * 16) : zero_bf16x8();
    }
  }
  // K^T for the dQ product: kt[d][key in tile]
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
    for (int j = 0; j < 8; ++j) sm.kt[(kk * 16 + hh * 8 + j) * S::KTP + w * 32 + li] = kf[kk][j];

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[db][i] = 0.f;
      dva[db][i] = 0.f;
    }

  for (int mb = t.m_lo; mb < t.m_hi; mb += kBwdBM) {
    __syncthreads();  // previous block fully consumed (and K^T staged)
    for (int c = threadIdx.x; c < kBwdBM * (D / 8); c += kThreads) {
      const int rr = c % kBwdBM, dc = c / kBwdBM;
      const int m = mb + rr;
      const bool ok = m < t.m_hi;
      const int64_t off = (int64_t)m * rs + (int64_t)h * D + dc * 8;
      const bf16x8 qv = ok ? load_bf16x8(q + off) : zero_bf16x8();
      const bf16x8 dv8 = ok ? load_bf16x8(d_o + off) : zero_bf16x8();
      store_bf16x8(&sm.q[rr * S::QP + dc * 8], qv);
      store_bf16x8(&sm.dO[rr * S::QP + dc * 8], dv8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sm.qt[(dc * 8 + j) * S::TP + rr] = qv[j];
        sm.dOt[(dc * 8 + j) * S::TP + rr] = dv8[j];
      }
    }
    if (threadIdx.x < kBwdBM) {
      const int rr = threadIdx.x;
      const int m = mb + rr;
      const bool ok = m < t.m_hi;
      sm.lse2[rr] = ok ? lse[(int64_t)h * n_local + m] * kLog2e : 0.f;
      sm.dlt[rr] = ok ? delta[(int64_t)h * n_local + m] : 0.f;
      sm.gq[rr] = ok ? m + (m < t.m_split ? t.dg_a : t.dg_b) : -1;
    }
    __syncthreads();

    if (wave_live) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
      const bf16* qa = &sm.q[li * S::QP + hh * 8];
      const bf16* da = &sm.dO[li * S::QP + hh * 8];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s = mfma32(load_bf16x8(qa + kk * 16), kf[kk], s);
        dp = mfma32(load_bf16x8(da + kk * 16), vf[kk], dp);
      }
      // Element i of this lane: query row 8*(i/4) + 4*hh + i%4, key my_key.
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int qr0 = i4 * 8 + hh * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[qr0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[qr0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i4 * 4 + j;
          const bool ok = key_ok && my_key <= sm.gq[qr0 + j];
          const float p = ok ? exp2f(fmaf(s[i], scale_log2, -l4[j])) : 0.f;
          const float dsv = ok ? p * (dp[i] - d4[j]) : 0.f;
          s[i] = p;
          dp[i] = dsv;
        }
      }
      // dV += P^T dO and dK += dS^T Q. k-step u covers query rows
      // 16u + (j/4)*8 + hh*4 + j%4 for slot j: accumulator entries u*8..u*8+7.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pa = to_bf16x8(s, u * 8);
        const bf16x8 dsa = to_bf16x8(dp, u * 8);
        const int qcol = 16 * u + hh * 4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16* dop = &sm.dOt[(db * 32 + li) * S::TP + qcol];
          dva[db] = mfma32(pa, concat4(load_bf16x4(dop), load_bf16x4(dop + 8)), dva[db]);
          const bf16* qp = &sm.qt[(db * 32 + li) * S::TP + qcol];
          dka[db] = mfma32(dsa, concat4(load_bf16x4(qp), load_bf16x4(qp + 8)), dka[db]);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = (i >> 2) * 8 + hh * 4 + (i & 3);
        sm.ds[qr * S::SP + w * 32 + li] = (bf16)dp[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = (i >> 2) * 8 + hh * 4 + (i & 3);
        sm.ds[qr * S::SP + w * 32 + li] = (bf16)0.f;
      }
    }
    __syncthreads();

    // dQ[queries, 32w .. 32w+31] += scale * dS (32 x 128 keys) K (128 keys x 32 dims)
    if (w < DB) {
      f32x16 dqa;
#pragma unroll
      for (int i = 0; i < 16; ++i) dqa[i] = 0.f;
      const bf16* dsa = &sm.ds[li * S::SP + hh * 8];
      const bf16* kta = &sm.kt[(w * 32 + li) * S::KTP + hh * 8];
#pragma unroll
      for (int kt = 0; kt < kBwdBN / 16; ++kt)
        dqa = mfma32(load_bf16x8(dsa + kt * 16), load_bf16x8(kta + kt * 16), dqa);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = (i >> 2) * 8 + hh * 4 + (i & 3);
        const int m = mb + qr;
        if (m < t.m_hi) unsafeAtomicAdd(dq + (int64_t)m * rs + (int64_t)h * D + w * 32 + li, dqa[i] * scale);
      }
    }
  }

  // dK (scaled) and dV rows of this wave's keys; lane li holds head dim db*32 + li.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = t.k0 + w * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
      if (key < t.k1) {
        const int64_t off = (int64_t)key * rs + (int64_t)h * D + db * 32 + li;
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
                        const float* delta, float* dq, float* dk, float* dv, int64_t n_local,
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
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_kernel<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  hipLaunchKernelGGL(attn_bwd_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), smem, stream,
                     tiles, H, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<const bf16*>(d_o), lse, delta, dq,
                     dk, dv, n_local, scale, scale * kLog2e, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                           const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, float* dq, float* dk,
                           float* dv, int64_t n_local, float scale, int32_t accumulate,
                           hipStream_t stream) {
  if (D == 128)
    return launch_bwd_d<128>(tiles, n_tiles, H, q, k, v, d_o, lse, delta, dq, dk, dv, n_local,
                             scale, accumulate, stream);
  if (D == 64)
    return launch_bwd_d<64>(tiles, n_tiles, H, q, k, v, d_o, lse, delta, dq, dk, dv, n_local,
                            scale, accumulate, stream);
  return hipErrorInvalidValue;
}

}  // namespace thdcp
