// Backward, key side: this rank's partial dK/dV over the full K/V ("[PyTorch]
// Add no-load-balance THD all-gather CP", sequence diagram: the dK/dV partials
// are unrestored for the reduce-scatter). dQ is computed by the query-major
// kernel in attn_bwd_dq.hip, so this kernel needs no atomics and every key row
// it owns is written by exactly one workgroup. Padding never enters a product:
// query rows that are not real tokens are not listed, key rows past the tile
// end are zeroed, and masked probabilities are selected to 0 (NaN-safe).
//
// gfx950 design: a workgroup of 4 or 8 waves owns 128 or 256 consecutive keys
// of one document, 32 per wave (two 16-key blocks), with the K fragments in
// registers and the V rows in LDS, and walks the local query rows that attend
// them in blocks of 32. Query blocks (Q, dO, LSE, delta) are double-buffered
// in LDS and the next block's global loads are in flight while the current
// one is computed; one barrier per block. Per block each wave computes with
// v_mfma_f32_16x16x32_bf16
//   S = Q K^T, dP = dO V^T          (A = Q / dO rows from LDS, B = K regs / V LDS)
//   P = exp(S - LSE), dS = P (dP - delta)
//   dV += P^T dO, dK += dS^T Q       (accumulators stay in registers)
// P and dS come out of the first products already in the A-operand layout of
// the last two; their B operands (dO and Q, sliced by column) are transposing
// LDS reads of the row-major tiles. Every Q / dO fragment read from LDS feeds
// both key blocks, so a wave reads 0.625 KB of LDS per MFMA (1 KB with 16 keys
// per wave, which made the LDS as busy as the MFMA pipe). At <= 256 registers
// per wave and ~75 KB of LDS per workgroup, two 4-wave workgroups share a CU
// (two waves per SIMD), and one workgroup's prologue and stores overlap the
// other's block loop. Plans whose query walks are long use one 8-wave
// workgroup per CU instead (~112 KB of LDS), which stages each query block
// once for twice the keys.
#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace thdcp {

namespace {

constexpr int kBM = 32;  // query rows per block (two 16-query M-blocks)
constexpr float kLog2e = 1.4426950408889634f;

template <int D, int WAVES>
struct BwdSmem {
  static constexpr int P = D + 16;     // Q / dO row pitch (bf16)
  bf16 q[2][kBM * P];
  bf16 dO[2][kBM * P];
  float lse2[2][kBM];
  float dlt[2][kBM];
  int32_t ghi[2][kBM];  // last key a query row attends (g + wr); -1 past the row range
  int32_t glo[2][kBM];  // first key (g - wl); read only for non-causal bands
  bf16 v[WAVES * 32 * P];  // the tile's V rows (wave w's keys at rows 32w..), pitch P
};

// BAND: the mask is a general band [g - wl, g + wr] (a lower-bound test
// per element); otherwise it is causal (key <= g only). WAVES: 4 (128-key
// tiles) or 8 (256-key tiles); two waves per SIMD either way.
template <int D, int WAVES, bool BAND>
__global__ void __launch_bounds__(WAVES * 64, 2)
attn_bwd_dkdv_kernel(const BwdTile* __restrict__ tiles, int32_t H, const bf16* __restrict__ q,
                     const bf16* __restrict__ k, const bf16* __restrict__ v,
                     const int32_t* __restrict__ kv_row, int32_t kv_sub, int32_t wl, int32_t wr,
                     const bf16* __restrict__ d_o,
                     const float* __restrict__ lse,
                     const float* __restrict__ delta, float* __restrict__ dk,
                     float* __restrict__ dv, int64_t n_local, float scale, float scale_log2,
                     int32_t accumulate) {
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int CPR = D / 8;
  constexpr int kThreads = WAVES * 64;
  constexpr int CHUNKS = kBM * CPR;                       // 16-byte chunks per block
  constexpr int CH = (CHUNKS + kThreads - 1) / kThreads;  // staging chunks per thread
  constexpr bool kPartial = CHUNKS % kThreads != 0;       // some threads stage nothing
  typedef BwdSmem<D, WAVES> S;
  constexpr int P = S::P;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  S& sm = *reinterpret_cast<S*>(smem_raw);

  const int tile_id = blockIdx.x / H;
  const int h = blockIdx.x - tile_id * H;
  const BwdTile t = tiles[tile_id];
  // Wave index, made wave-uniform explicitly so it and the LDS addresses
  // derived from it live in scalar registers.
  const int w = wave_uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int G = lane >> 4;
  const int64_t rs = (int64_t)H * D;
  const int64_t head_off = (int64_t)h * D;

  // Key j sits at row j - kv_sub of K/V and dK/dV (global order, or one
  // rank's block of it) or at row kv_row[j] - kv_sub (rank-major, or one
  // rank's block of it: the restore and the unrestore fused into these loads
  // and stores).
  auto key_row = [&](int key) -> int64_t {
    return (int64_t)(kv_row ? kv_row[key] : key) - kv_sub;
  };
  // Lane l16 of key block nk holds key t.k0 + 32w + 16nk + l16: the column of
  // S / dP and the row of the dV / dK A operand.
  // This wave's keys: [wave_kmin, wave_kmax], all below the tile end or not.
  const int wave_kmin = t.k0 + w * 32, wave_kmax = wave_kmin + 31;
  const bool wave_keys_ok = wave_kmax < t.k1;
  int my_key[2];
  bool key_ok[2];
  bf16x8 kf[2][KS];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk) {
    my_key[nk] = t.k0 + w * 32 + nk * 16 + l16;
    key_ok[nk] = my_key[nk] < t.k1;
    const int64_t off = key_row(min(my_key[nk], t.k1 - 1)) * rs + head_off + G * 8;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      kf[nk][kk] = key_ok[nk] ? load_bf16x8(k + off + kk * 32) : zero_bf16x8();
  }
  // V rows of this wave's 32 keys into LDS (only this wave reads them; rows
  // past the tile end are 0): 32 rows x CPR 16-byte chunks over 64 lanes.
#pragma unroll
  for (int j = 0; j < 32 * CPR / 64; ++j) {
    const int c = lane + j * 64;
    const int rr = c / CPR, dc = c - rr * CPR;
    const int key = t.k0 + w * 32 + rr;
    const bf16x8 x = key < t.k1 ? load_bf16x8(v + key_row(key) * rs + head_off + dc * 8)
                                : zero_bf16x8();
    *reinterpret_cast<bf16x8*>(&sm.v[(w * 32 + rr) * P + dc * 8]) = x;
  }
  f32x4 dka[2][NB], dva[2][NB];
#pragma unroll
  for (int nk = 0; nk < 2; ++nk)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dka[nk][nb][i] = 0.f;
        dva[nk][nb][i] = 0.f;
      }

  // Per-thread staging slots: chunk c = threadIdx + j*kThreads is row c/CPR,
  // 16-byte column c%CPR of the query block. When the chunks do not fill the
  // last round (head dim 64 over 8 waves), the waves past them stage nothing
  // in it (a whole-wave condition: CHUNKS is a multiple of 64).
  const bool stages_last = !kPartial || (int)threadIdx.x + (CH - 1) * kThreads < CHUNKS;
  auto has_chunk = [&](int j) { return j < CH - 1 || stages_last; };
  uint32_t goff[CH];
  int soff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int c = has_chunk(j) ? threadIdx.x + j * kThreads : 0;
    const int rr = c / CPR, dc = c - rr * CPR;
    goff[j] = (uint32_t)(rr * rs * 2 + dc * 16);
    soff[j] = rr * P + dc * 8;
  }
  // Loads are buffer loads whose descriptors end at row m_hi (later rows read
  // 0), so they need no branch; nothing is computed from them until they are
  // written to LDS after the current block's MFMAs, so they stay in flight.
  u32x4 qreg[CH], dreg[CH];
  float lreg = 0.f, dlreg = 0.f;
  int hreg = -1, loreg = 0;
  auto load_block = [&](int mb) {
    const int64_t base = (int64_t)mb * rs + head_off;
    const uint32_t bytes = (uint32_t)((int64_t)(t.m_hi - mb) * rs * 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + base, bytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(d_o + base, bytes);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (has_chunk(j)) {
        qreg[j] = buffer_load16(rq, goff[j]);
        dreg[j] = buffer_load16(rd, goff[j]);
      }
    }
    if (wave_uniform(w) == 0) {  // wave 0 fetches the block's per-row scalars
      const int64_t row = (int64_t)h * n_local + mb;
      const uint32_t rbytes = (uint32_t)(t.m_hi - mb) * 4u;
      lreg = buffer_load_f32(make_rsrc(lse + row, rbytes), (uint32_t)lane * 4u);
      dlreg = buffer_load_f32(make_rsrc(delta + row, rbytes), (uint32_t)lane * 4u);
      const int m = mb + lane;
      const int g = m + (m < t.m_split ? t.dg_a : t.dg_b);
      hreg = m < t.m_hi ? g + wr : -1;
      if constexpr (BAND) loreg = g - wl;
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (has_chunk(j)) {
        *reinterpret_cast<u32x4*>(&sm.q[buf][soff[j]]) = qreg[j];
        *reinterpret_cast<u32x4*>(&sm.dO[buf][soff[j]]) = dreg[j];
      }
    }
    if (wave_uniform(w) == 0 && lane < kBM) {
      sm.lse2[buf][lane] = lreg * kLog2e;
      sm.dlt[buf][lane] = dlreg;
      sm.ghi[buf][lane] = hreg;
      if constexpr (BAND) sm.glo[buf][lane] = loreg;
    }
  };

  const int nblocks = (t.m_hi - t.m_lo + kBM - 1) / kBM;
  load_block(t.m_lo);
  store_block(0);
  wait_vmem();  // K fragments and V rows have landed: the loop's MFMAs never wait on loads
  __syncthreads();

  for (int it = 0; it < nblocks; ++it) {
    const int mb = t.m_lo + it * kBM;
    const int cur = it & 1;
    const bool has_next = it + 1 < nblocks;
    if (has_next) load_block(mb + kBM);

    // S and dP, [16-query M-block qm][key block nk]; element i of s[qm][nk] is
    // query row qm*16 + 4*G + i, key my_key[nk]. dP accumulates from -delta of
    // its row, so the products leave dP - delta and dS = P (dP - delta) is one
    // multiply.
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int qm = 0; qm < 2; ++qm) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[cur][qm * 16 + G * 4]);
#pragma unroll
      for (int nk = 0; nk < 2; ++nk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[qm][nk][i] = 0.f;
          dp[qm][nk][i] = -d4[i];
        }
    }
    if constexpr (WAVES == 8) {
      // Steps n = 2kk + qm (k-step kk, 16-query block qm). The Q / dO
      // fragments of step n + 1, and at a new k-step its two V fragments, are
      // read while step n's MFMAs run; the scheduling barriers keep them there
      // (left to the compiler, each MFMA pair waited on its own reads; -2% on
      // 256-key tiles; even on 128-key tiles, where a band instance spills).
      bf16x8 aqr[2], adr[2], vbr[2][2];
      auto fetch = [&](int n) {
        const int kk = n >> 1, qm = n & 1;
        if (qm == 0) {
#pragma unroll
          for (int nk = 0; nk < 2; ++nk)
            vbr[kk & 1][nk] = load_bf16x8(&sm.v[(w * 32 + nk * 16 + l16) * P + kk * 32 + G * 8]);
        }
        const int o = (qm * 16 + l16) * P + kk * 32 + G * 8;
        aqr[n & 1] = load_bf16x8(&sm.q[cur][o]);
        adr[n & 1] = load_bf16x8(&sm.dO[cur][o]);
      };
      fetch(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < 2 * KS; ++n) {
        if (n + 1 < 2 * KS) fetch(n + 1);
        const int kk = n >> 1, qm = n & 1;
#pragma unroll
        for (int nk = 0; nk < 2; ++nk) {
          s[qm][nk] = mfma16(aqr[n & 1], kf[nk][kk], s[qm][nk]);
          dp[qm][nk] = mfma16(adr[n & 1], vbr[kk & 1][nk], dp[qm][nk]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        bf16x8 vb[2];
#pragma unroll
        for (int nk = 0; nk < 2; ++nk)
          vb[nk] = load_bf16x8(&sm.v[(w * 32 + nk * 16 + l16) * P + kk * 32 + G * 8]);
#pragma unroll
        for (int qm = 0; qm < 2; ++qm) {
          const int o = (qm * 16 + l16) * P + kk * 32 + G * 8;
          const bf16x8 aq = load_bf16x8(&sm.q[cur][o]);
          const bf16x8 ad = load_bf16x8(&sm.dO[cur][o]);
#pragma unroll
          for (int nk = 0; nk < 2; ++nk) {
            s[qm][nk] = mfma16(aq, kf[nk][kk], s[qm][nk]);
            dp[qm][nk] = mfma16(ad, vb[nk], dp[qm][nk]);
          }
        }
      }
    }
    // P = exp2(S * scale_log2 - LSE_2) and dS = P (dP - delta). A masked
    // element takes exponent -inf, so P = 0 and dS = 0 with no branch (dP is
    // finite: rows past the range and keys past the tile load as zeros). The
    // per-element mask is only evaluated on blocks that need it: a block whose
    // rows are all real and whose bands hold all of this wave's keys (rows'
    // band ends rise with the row, and are -1 past the range) skips it.
    const int blk_hi = min(sm.ghi[cur][0], sm.ghi[cur][kBM - 1]);
    bool inside = wave_keys_ok && blk_hi >= wave_kmax;
    if constexpr (BAND) inside = inside && sm.glo[cur][kBM - 1] <= wave_kmin;
    const bool masked = wave_uniform(!inside) != 0;
#pragma unroll
    for (int qm = 0; qm < 2; ++qm) {
      const int qr0 = qm * 16 + G * 4;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[cur][qr0]);
      if (masked) {
        const i32x4 hi4 = *reinterpret_cast<const i32x4*>(&sm.ghi[cur][qr0]);
        i32x4 lo4 = {0, 0, 0, 0};
        if constexpr (BAND) lo4 = *reinterpret_cast<const i32x4*>(&sm.glo[cur][qr0]);
#pragma unroll
        for (int nk = 0; nk < 2; ++nk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bool ok = key_ok[nk] & (my_key[nk] <= hi4[i]);
            if constexpr (BAND) ok &= my_key[nk] >= lo4[i];
            s[qm][nk][i] = ok ? fmaf(s[qm][nk][i], scale_log2, -l4[i]) : -INFINITY;
          }
      } else {
#pragma unroll
        for (int nk = 0; nk < 2; ++nk)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[qm][nk][i] = fmaf(s[qm][nk][i], scale_log2, -l4[i]);
      }
#pragma unroll
      for (int nk = 0; nk < 2; ++nk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(s[qm][nk][i]);
          s[qm][nk][i] = p;
          dp[qm][nk][i] = p * dp[qm][nk][i];
        }
    }
    // dV += P^T dO, dK += dS^T Q over the block's 32 queries (one k-step):
    // slot j of this lane is query (j/4)*16 + 4*G + j%4. Each transposed dO
    // / Q read feeds both key blocks.
    bf16x8 pa[2], dsa[2];
#pragma unroll
    for (int nk = 0; nk < 2; ++nk) {
      pa[nk] = pack8(s[0][nk], s[1][nk]);
      dsa[nk] = pack8(dp[0][nk], dp[1][nk]);
    }
    const int o1 = (G * 4 + (l16 >> 2)) * P + 4 * (l16 & 3);
    const int o2 = o1 + 16 * P;
    auto read_b = [&](const bf16* tile, int nb) {
      return concat4(lds_read_tr4(tile + o1 + nb * 16), lds_read_tr4(tile + o2 + nb * 16));
    };
    // The B operands of head-dim block nb + 1 are read while block nb's MFMAs
    // run (without it every MFMA pair waited on its own reads; -3..-6%).
    // Raised wave priority over these products lets this wave's MFMAs issue
    // ahead of the softmax of the other workgroup's wave on the SIMD.
    __builtin_amdgcn_s_setprio(1);
    bf16x8 bdo_next = read_b(sm.dO[cur], 0), bq_next = read_b(sm.q[cur], 0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bf16x8 bdo = bdo_next, bq = bq_next;
      if (nb + 1 < NB) {
        bdo_next = read_b(sm.dO[cur], nb + 1);
        bq_next = read_b(sm.q[cur], nb + 1);
      }
      dva[0][nb] = mfma16(pa[0], bdo, dva[0][nb]);
      dva[1][nb] = mfma16(pa[1], bdo, dva[1][nb]);
      dka[0][nb] = mfma16(dsa[0], bq, dka[0][nb]);
      dka[1][nb] = mfma16(dsa[1], bq, dka[1][nb]);
    }
    __builtin_amdgcn_s_setprio(0);
    if (has_next) store_block(cur ^ 1);
    __syncthreads();
  }

  // dK (scaled) and dV rows of this wave's keys; lane holds head dim nb*16 + l16
  // for keys 16*nk + 4*G + i of the wave's 32.
#pragma unroll
  for (int nk = 0; nk < 2; ++nk) {
    int64_t out_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = t.k0 + w * 32 + nk * 16 + G * 4 + i;
      out_row[i] = key < t.k1 ? key_row(key) : -1;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (out_row[i] >= 0) {
          const int64_t off = out_row[i] * rs + head_off + nb * 16 + l16;
          const float kval = dka[nk][nb][i] * scale;
          const float vval = dva[nk][nb][i];
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
}

template <int D, int WAVES, bool BAND>
hipError_t launch_bwd_d(const BwdTile* tiles, int32_t n_tiles, int32_t H, const void* q,
                        const void* k, const void* v, const int32_t* kv_row, int32_t kv_sub,
                        Band band, const void* d_o, const float* lse, const float* delta, float* dk,
                        float* dv, int64_t n_local, float scale, int32_t accumulate,
                        hipStream_t stream) {
  const int64_t blocks = (int64_t)n_tiles * H;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const size_t smem = sizeof(BwdSmem<D, WAVES>);
  // The dynamic-LDS limit is a per-device function attribute: set it once per device.
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load() & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, WAVES, BAND>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit);
  }
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, WAVES, BAND>), dim3((unsigned)blocks),
                     dim3(WAVES * 64),
                     smem, stream, tiles, H, static_cast<const bf16*>(q),
                     static_cast<const bf16*>(k), static_cast<const bf16*>(v), kv_row, kv_sub,
                     band.wl, band.wr, static_cast<const bf16*>(d_o),
                     lse, delta, dk, dv, n_local, scale, scale * kLog2e, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_dkdv(const BwdTile* tiles, int32_t n_tiles, int32_t H, int32_t D,
                                int32_t keys, const void* q, const void* k, const void* v, KvRows kv,
                                Band band, const void* d_o, const float* lse,
                                const float* delta, float* dk, float* dv, int64_t n_local,
                                float scale, int32_t accumulate, hipStream_t stream) {
  const int32_t sub = (int32_t)kv.sub;
#define THDCP_DKDV(DD, WW, BB)                                                                \
  return launch_bwd_d<DD, WW, BB>(tiles, n_tiles, H, q, k, v, kv.map, sub, band, d_o, lse,     \
                                  delta, dk, dv, n_local, scale, accumulate, stream)
  if (keys != kBwdBN && keys != kBwdBNLong) return hipErrorInvalidValue;
  const bool wide = keys == kBwdBNLong;
  if (D == 128 && band.causal) {
    if (wide) THDCP_DKDV(128, 8, false);
    THDCP_DKDV(128, 4, false);
  }
  if (D == 128) {
    if (wide) THDCP_DKDV(128, 8, true);
    THDCP_DKDV(128, 4, true);
  }
  if (D == 64 && band.causal) {
    if (wide) THDCP_DKDV(64, 8, false);
    THDCP_DKDV(64, 4, false);
  }
  if (D == 64) {
    if (wide) THDCP_DKDV(64, 8, true);
    THDCP_DKDV(64, 4, true);
  }
#undef THDCP_DKDV
  return hipErrorInvalidValue;
}

}  // namespace thdcp
