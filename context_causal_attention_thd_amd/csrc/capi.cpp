// C ABI of libthdcp: argument checks, by-value padding detection, the rank
// plan, and dispatch of the gfx950 kernels on the caller's stream.
//
// Pages cited (title and section):
//   [AG]  "[PyTorch] Add no-load-balance THD all-gather CP"
//   [A2A] "[PyTorch] Extend no-load-balance CP to the a2a comm type"
//   [PAD] "[PyTorch][Attention] THD P2P context-parallel regression when padded
//          cu_seqlens are value-equal but not object-identical"
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include "thdcp.h"
#include "internal.h"

using namespace thdcp;

namespace {

thread_local std::string g_last_error;

thdcp_status_t fail(thdcp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

thdcp_status_t ok() {
  g_last_error.clear();
  return THDCP_OK;
}

thdcp_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(THDCP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// Error reporting for the library's other translation units (not exported).
thdcp_status_t thdcp::report_error(thdcp_status_t st, const char* msg) {
  return fail(st, "%s", msg);
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Layout rules ([AG] "Why", "Scope and constraints"; [A2A] body) and padding
// by value ([PAD] "Expected behavior").
thdcp_status_t check_layout(const int32_t* cu, const int32_t* cup, int32_t B, int64_t T,
                            int32_t cp, int32_t rank, int32_t strategy, int32_t wl, int32_t wr,
                            int32_t pad_flag, int32_t* padding_out) {
  if (!cup) return fail(THDCP_ERR_ARG, "cu_seqlens_padded_host is NULL");
  if (B < 0) return fail(THDCP_ERR_ARG, "B must be >= 0 (got %d)", B);
  if (cp < 1) return fail(THDCP_ERR_ARG, "cp_size must be >= 1 (got %d)", cp);
  if (rank < 0 || rank >= cp) return fail(THDCP_ERR_ARG, "rank %d outside [0, %d)", rank, cp);
  if (strategy != THDCP_DUAL_CHUNK_SWAP && strategy != THDCP_NO_LOAD_BALANCE)
    return fail(THDCP_ERR_ARG, "unknown strategy %d", strategy);
  if (wl < -1 || wr < -1)
    return fail(THDCP_ERR_ARG, "window_size (%d, %d): each side must be >= 0 or -1 (no bound)",
                wl, wr);
  if (T < 0 || T > INT32_MAX / 2) return fail(THDCP_ERR_ARG, "T=%lld out of range", (long long)T);
  if (pad_flag < -1 || pad_flag > 1) return fail(THDCP_ERR_ARG, "pad_between_seqs must be -1, 0 or 1");
  if (cup[0] != 0 || (cu && cu[0] != 0))
    return fail(THDCP_ERR_LAYOUT, "cumulative sequence lengths must start at 0");
  bool padding = false;
  for (int32_t i = 0; i < B; ++i) {
    const int64_t p = (int64_t)cup[i + 1] - cup[i];
    const int64_t n = cu ? (int64_t)cu[i + 1] - cu[i] : p;
    if (p < 0 || n < 0)
      return fail(THDCP_ERR_LAYOUT, "cumulative sequence lengths decrease at doc %d", i);
    if (n > p)
      return fail(THDCP_ERR_LAYOUT, "doc %d: actual length %lld exceeds padded length %lld", i,
                  (long long)n, (long long)p);
    if (strategy == THDCP_DUAL_CHUNK_SWAP && p % (2 * (int64_t)cp) != 0)
      return fail(THDCP_ERR_LAYOUT,
                  "DUAL_CHUNK_SWAP: padded length %lld of doc %d is not divisible by "
                  "2*cp_size=%d", (long long)p, i, 2 * cp);
    if (n != p) padding = true;
  }
  if ((int64_t)cup[B] > T)
    return fail(THDCP_ERR_LAYOUT, "cu_seqlens_padded[B]=%d exceeds T=%lld", cup[B], (long long)T);
  if (strategy == THDCP_DUAL_CHUNK_SWAP && (int64_t)cup[B] != T)
    return fail(THDCP_ERR_LAYOUT, "DUAL_CHUNK_SWAP needs T == cu_seqlens_padded[B]");
  if (T % cp != 0)
    return fail(THDCP_ERR_LAYOUT, "T=%lld is not divisible by cp_size=%d", (long long)T, cp);
  if ((int64_t)cup[B] < T) padding = true;
  if (pad_flag == 0 && padding)
    return fail(THDCP_ERR_ARG,
                "pad_between_seqs=0 but the sequence lengths show padding between sequences");
  if (padding_out) *padding_out = padding ? 1 : 0;
  return ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------
struct thdcp_plan {
  thdcp_attn_desc desc;
  Band band{kUnbounded, 0, true};  // the mask's key band (causal by default)
  std::vector<int32_t> cu, cup;
  int64_t n_local = 0;
  float scale = 0.f;
  int32_t padding = 0;
  int64_t pairs = 0, touched = 0;
  std::vector<int32_t> local_seqlens;
  std::vector<FwdTile> fwd;
  std::vector<BwdTile> bwd;
  std::vector<ZeroRange> zero;
  // kv_row[g] = rank-major position of global row g, built when rank-major
  // order differs from global order (DUAL_CHUNK_SWAP, cp_size > 1) and either
  // the all-gather calls take rank-major K/V (kv_mapped) or P2P steps read
  // one rank's local K/V block through it.
  bool kv_mapped = false;
  std::vector<int32_t> kv_row;
  // P2P ring steps (desc.p2p): per source rank s, forward tiles (one per
  // query tile, holding the keys rank s has), key tiles over rank s's keys,
  // and rank s's rows no local query attends. Concatenated over s.
  struct Step {
    int32_t fwd0, n_fwd, bwd0, n_bwd, zero0, n_zero;
    int64_t untouched;
  };
  std::vector<Step> steps;
  std::vector<FwdTile> step_fwd;
  std::vector<BwdTile> step_bwd;
  std::vector<ZeroRange> step_zero;
  // Split key walks of the all-gather forward / dQ tiles: groups (one counter
  // per group and head) and scratch slots (one per part and head).
  int32_t split_groups = 0, split_slots = 0, split_tiles = 0;
  // Query rows per forward / dQ tile and keys per dK/dV tile: kFwdBMLong and
  // kBwdBNLong when the average query walks at least kLongWalk keys
  // (all-gather plans), else kFwdBM and kBwdBN.
  int32_t fwd_rows = kFwdBM;
  int32_t bwd_keys = kBwdBN;
  // Transposed-V forward (256-row tiles, head dim 128): V^T of all T keys at
  // off_vt in the workspace, key pitch vt_pitch, written by cp_attn_fwd.
  bool fwd_vt = false;
  int32_t vt_pitch = 0;
  size_t off_vt = 0;
  std::vector<char> blob;  // host image of the device tables (and zeroed counters)
  size_t off_fwd = 0, off_bwd = 0, off_zero = 0, off_kvrow = 0, ws_bytes = 0;
  size_t off_sfwd = 0, off_sbwd = 0, off_szero = 0, off_cnt = 0, off_part = 0;
  char* ws_dev = nullptr;  // caller's workspace after upload
};

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Keys a real query at global row g of a document with real rows [a, e)
// attends: the band [g - wl, g + wr] inside [a, e) (causal: [a, g]).
int64_t key_lo(const Band& b, int64_t a, int64_t g) { return std::max<int64_t>(a, g - b.wl); }
int64_t key_hi(const Band& b, int64_t e, int64_t g) { return std::min<int64_t>(e - 1, g + b.wr); }

struct Segment {  // consecutive local rows holding consecutive global rows of one document
  int64_t m0, g0, len;
  int64_t a, e;   // document start and end of its real tokens
  int32_t doc;    // -1: buffer tail (no document)
};

std::vector<Segment> build_segments(const thdcp_plan& p, int64_t r) {
  const auto& d = p.desc;
  const int64_t cp = d.cp_size;
  std::vector<Segment> segs;
  if (d.strategy == THDCP_DUAL_CHUNK_SWAP) {
    // [AG] "Why": 2*cp_size chunks per document; rank r holds chunks r and
    // 2*cp_size-1-r, document-major, local offset of doc i = cup[i]/cp_size.
    for (int32_t i = 0; i < d.B; ++i) {
      const int64_t P = p.cup[i + 1] - p.cup[i];
      const int64_t c = P / (2 * cp);
      if (c == 0) continue;
      const int64_t a = p.cup[i], e = a + (p.cu[i + 1] - p.cu[i]);
      const int64_t mdoc = a / cp;
      segs.push_back({mdoc, a + r * c, c, a, e, i});
      segs.push_back({mdoc + c, a + (2 * cp - 1 - r) * c, c, a, e, i});
    }
  } else {
    // [AG] "What changed"; [A2A] body: rank r holds [r*s_local, (r+1)*s_local).
    const int64_t s = d.T / cp, lo = r * s, hi = lo + s;
    for (int32_t i = 0; i < d.B; ++i) {
      const int64_t x0 = std::max<int64_t>(lo, p.cup[i]), x1 = std::min<int64_t>(hi, p.cup[i + 1]);
      if (x1 <= x0) continue;
      const int64_t a = p.cup[i], e = a + (p.cu[i + 1] - p.cu[i]);
      segs.push_back({x0 - lo, x0, x1 - x0, a, e, i});
    }
    const int64_t t0 = std::max<int64_t>(lo, p.cup[d.B]);
    if (t0 < hi) segs.push_back({t0 - lo, t0, hi - t0, t0, t0, -1});
  }
  return segs;
}

// Key tiles of a forward tile, the cost the LPT order sorts by.
int64_t fwd_cost(const FwdTile& t) {
  const int64_t n0 = t.ke0 > t.ks0 ? (t.ke0 - t.ks0 + kFwdBN - 1) / kFwdBN : 0;
  const int64_t n1 = t.ke1 > t.ks1 ? (t.ke1 - t.ks1 + kFwdBN - 1) / kFwdBN : 0;
  return n0 + n1;
}

// Longest first (LPT order over the workgroup queue), stable.
template <typename Tile, typename Cost>
std::vector<Tile> lpt_order(const std::vector<Tile>& tiles, Cost cost) {
  std::vector<size_t> order(tiles.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t x, size_t y) { return cost(tiles[x]) > cost(tiles[y]); });
  std::vector<Tile> sorted;
  sorted.reserve(tiles.size());
  for (size_t i : order) sorted.push_back(tiles[i]);
  return sorted;
}

// Split key walks. A forward or dQ launch runs one workgroup per (tile,
// head), and the chip holds kConcurrentWGs of them at once. When that grid
// barely fills the chip and the walks are very uneven (few heads over long
// causal documents: the last query tile of a document walks all of it), the
// longest walks, not the total work, set the launch's duration. Then every
// walk longer than the balanced load (the total key tiles over the
// concurrent workgroups) is divided into parts of consecutive key tiles no
// longer than that load, at most max_parts (kMaxParts when 0). Measured on
// MI355X, splitting pays (forward -17..20%, dQ -25..28%) when the longest
// walk is twice the balanced load, and does not at 1.25 and 1.5 times, where
// the tail's workgroups already run faster on emptied CUs and each part adds
// a prologue; hence the kSplitImbalance threshold for the automatic choice
// (a forced max_parts >= 2 splits from the balanced load on). Returns the
// table in LPT order.
// 256 CUs x 2 forward (or dQ) workgroups of 128-row tiles, x 1 of 256-row tiles
constexpr int64_t kConcurrentWGs = 512;
constexpr int64_t kMinPartTiles = 6;     // shorter parts do not repay their merge
constexpr double kSplitImbalance = 1.75;
constexpr int32_t kMaxParts = 8;

std::vector<FwdTile> split_walks(const std::vector<FwdTile>& tiles, int32_t H, int32_t rows,
                                 int32_t max_parts, int32_t* n_groups, int32_t* n_slots,
                                 int32_t* n_split) {
  int64_t total = 0;
  for (const FwdTile& t : tiles) total += fwd_cost(t);
  total *= H;
  const int64_t wgs = kConcurrentWGs * kFwdBM / rows;
  const int64_t target = std::max<int64_t>(kMinPartTiles, (total + wgs - 1) / wgs);
  int64_t longest = 0;
  for (const FwdTile& t : tiles) longest = std::max(longest, fwd_cost(t));
  int32_t cap = max_parts == 0 ? kMaxParts : std::min(max_parts, kMaxParts);
  if (max_parts == 0 && (double)longest < kSplitImbalance * (double)target) cap = 1;
  std::vector<FwdTile> out;
  int32_t groups = 0, slots = 0;
  for (const FwdTile& t : tiles) {
    const int64_t c = fwd_cost(t);
    const int32_t np = (int32_t)std::min<int64_t>(cap, (c + target - 1) / target);
    if (np < 2) {
      FwdTile u = t;
      u.part = 0;
      u.nparts = 1;
      u.slot = u.group = 0;
      out.push_back(u);
      continue;
    }
    // key tiles of the walk: n0 of [ks0, ke0), then those of [ks1, ke1)
    const int64_t n0 = t.ke0 > t.ks0 ? (t.ke0 - t.ks0 + kFwdBN - 1) / kFwdBN : 0;
    for (int32_t part = 0; part < np; ++part) {
      const int64_t a = c * part / np, b = c * (part + 1) / np;  // key tiles [a, b)
      FwdTile u = t;
      if (a < n0) {
        u.ks0 = (int32_t)(t.ks0 + a * kFwdBN);
        u.ke0 = (int32_t)std::min<int64_t>(t.ke0, t.ks0 + std::min(b, n0) * kFwdBN);
      } else {
        u.ks0 = u.ke0 = 0;
      }
      if (b > n0) {
        u.ks1 = (int32_t)(t.ks1 + (std::max(a, n0) - n0) * kFwdBN);
        u.ke1 = (int32_t)std::min<int64_t>(t.ke1, t.ks1 + (b - n0) * kFwdBN);
      } else {
        u.ks1 = u.ke1 = 0;
      }
      u.part = part;
      u.nparts = np;
      u.slot = slots;
      u.group = groups;
      out.push_back(u);
    }
    ++groups;
    slots += np;
  }
  *n_groups = groups;
  *n_slots = slots;
  *n_split = groups;
  return lpt_order(out, [](const FwdTile& t) { return fwd_cost(t); });
}

// A document's real local rows: runs of consecutive local rows holding
// consecutive global rows (one per DUAL_CHUNK_SWAP chunk, ascending in g).
struct DocRows {
  struct Run {
    int64_t m0, g0, n;
  };
  int32_t doc;
  int64_t a, e, gmax, m_hi, split, dga, dgb;
  std::vector<Run> runs;
};

std::vector<DocRows> doc_rows(const std::vector<Segment>& segs) {
  std::vector<DocRows> out;
  for (size_t si = 0; si < segs.size();) {
    const int32_t doc = segs[si].doc;
    size_t sj = si;
    while (sj < segs.size() && segs[sj].doc == doc && doc >= 0) ++sj;
    if (doc < 0) {
      ++si;
      continue;
    }
    DocRows dr{};
    dr.doc = doc;
    for (size_t k = si; k < sj; ++k) {
      const Segment& s = segs[k];
      const int64_t nv = std::max<int64_t>(0, std::min(s.g0 + s.len, s.e) - s.g0);
      if (nv > 0) dr.runs.push_back({s.m0, s.g0, nv});
    }
    dr.a = segs[si].a;
    dr.e = segs[si].e;
    si = sj;
    if (dr.runs.empty()) continue;
    const DocRows::Run& last = dr.runs.back();
    dr.gmax = last.g0 + last.n - 1;
    dr.m_hi = last.m0 + last.n;
    dr.split = dr.runs.size() > 1 ? dr.runs[1].m0 : dr.m_hi;
    dr.dga = dr.runs[0].g0 - dr.runs[0].m0;
    dr.dgb = dr.runs.size() > 1 ? dr.runs[1].g0 - dr.runs[1].m0 : dr.dga;
    out.push_back(std::move(dr));
  }
  return out;
}

// Key tiles of `keys` keys over [lo, hi) of one document; each lists the
// contiguous local query range that can attend it: real rows with
// g + wr >= k0 and g - wl <= k1 - 1 (causal: the rows with g >= k0). Local
// rows of a document ascend in g, so that range is contiguous.
void add_key_tiles(const DocRows& dr, const Band& band, int64_t keys, int64_t lo, int64_t hi,
                   std::vector<BwdTile>& out) {
  for (int64_t k0 = lo; k0 < hi; k0 += keys) {
    const int64_t k1 = std::min<int64_t>(k0 + keys, hi);
    const int64_t gfirst = k0 - band.wr, glast = k1 - 1 + (int64_t)band.wl;
    int64_t m_lo = -1;  // first local row with g >= gfirst
    for (const DocRows::Run& rn : dr.runs) {
      if (gfirst <= rn.g0 + rn.n - 1) {
        m_lo = rn.m0 + std::max<int64_t>(0, gfirst - rn.g0);
        break;
      }
    }
    int64_t m_hi = m_lo;  // one past the last local row with g <= glast
    for (auto it = dr.runs.rbegin(); it != dr.runs.rend(); ++it) {
      if (it->g0 <= glast) {
        m_hi = it->m0 + std::min<int64_t>(it->n, glast - it->g0 + 1);
        break;
      }
    }
    BwdTile t{};
    t.k0 = (int32_t)k0;
    t.k1 = (int32_t)k1;
    t.m_lo = (int32_t)m_lo;
    t.m_hi = (int32_t)m_hi;
    t.m_split = (int32_t)dr.split;
    t.dg_a = (int32_t)dr.dga;
    t.dg_b = (int32_t)dr.dgb;
    out.push_back(t);
  }
}

// Rows of the sorted ranges `own` not covered by the sorted ranges `touched`,
// with the running count of such rows before each range.
std::vector<ZeroRange> untouched_ranges(const std::vector<std::pair<int64_t, int64_t>>& own,
                                        const std::vector<std::pair<int64_t, int64_t>>& touched) {
  std::vector<ZeroRange> out;
  int64_t before = 0;
  size_t ti = 0;
  for (const auto& o : own) {
    int64_t cur = o.first;
    while (ti < touched.size() && touched[ti].second <= cur) ++ti;
    for (size_t tj = ti; tj < touched.size() && touched[tj].first < o.second; ++tj) {
      if (touched[tj].first > cur) {
        out.push_back({(int32_t)cur, (int32_t)touched[tj].first, (int32_t)before, 0});
        before += touched[tj].first - cur;
      }
      cur = std::max(cur, touched[tj].second);
    }
    if (cur < o.second) {
      out.push_back({(int32_t)cur, (int32_t)o.second, (int32_t)before, 0});
      before += o.second - cur;
    }
  }
  return out;
}

// Keys that rank `src` holds inside document `doc`, as at most two ascending
// global ranges: its DUAL_CHUNK_SWAP chunks src and 2*cp_size-1-src ([AG]
// "Why"), or its NO_LOAD_BALANCE range [src*s_local, (src+1)*s_local) ([AG]
// "What changed"), clipped to the document.
int key_ranges_of(const thdcp_plan& p, int32_t doc, int64_t src, int64_t (&lo)[2],
                  int64_t (&hi)[2]) {
  const auto& d = p.desc;
  const int64_t cp = d.cp_size;
  const int64_t a = p.cup[doc], b = p.cup[doc + 1];
  if (d.strategy == THDCP_DUAL_CHUNK_SWAP) {
    const int64_t c = (b - a) / (2 * cp);
    lo[0] = a + src * c;
    hi[0] = lo[0] + c;
    lo[1] = a + (2 * cp - 1 - src) * c;
    hi[1] = lo[1] + c;
    return 2;
  }
  const int64_t sl = d.T / cp;
  lo[0] = std::max<int64_t>(a, src * sl);
  hi[0] = std::min<int64_t>(b, (src + 1) * sl);
  return 1;
}

void build_plan(thdcp_plan& p) {
  const auto& d = p.desc;
  const std::vector<Segment> segs = build_segments(p, d.rank);

  p.local_seqlens.assign(d.B, 0);
  p.pairs = 0;
  for (const Segment& s : segs) {
    if (s.doc < 0) continue;
    const int64_t nvalid = std::max<int64_t>(0, std::min(s.g0 + s.len, s.e) - s.g0);
    p.local_seqlens[s.doc] += (int32_t)nvalid;
    if (p.band.causal) {
      // sum over real rows g in [g0, g0+nvalid) of (g - a + 1)
      const int64_t f = s.g0 - s.a + 1;
      p.pairs += nvalid * f + nvalid * (nvalid - 1) / 2;
    } else {
      for (int64_t g = s.g0; g < s.g0 + nvalid; ++g)
        p.pairs += key_hi(p.band, s.e, g) - key_lo(p.band, s.a, g) + 1;
    }
  }

  // Tile sizes. 256-row query tiles (8 waves of 32 rows, one workgroup per
  // CU) stage each K/V tile once for twice the queries and feed two MFMAs per
  // LDS fragment, and 256-key dK/dV tiles (8 waves, one workgroup per CU)
  // stage each query block once for twice the keys, but both keep one
  // workgroup per CU instead of two, which pays only where walks are long
  // enough to hide each workgroup's start. Measured on MI355X, one
  // 75600-token document: forward -5%, dQ even, dK/dV -5..-6%; shares of
  // documents of a few thousand tokens: 5-15% slower. P2P steps walk one
  // rank's keys each and keep the small tiles.
  constexpr int64_t kLongWalk = 4096;
  const bool long_walks = !d.p2p && p.pairs >= kLongWalk * std::max<int64_t>(1, p.n_local);
  p.fwd_rows = long_walks ? kFwdBMLong : kFwdBM;
  p.bwd_keys = long_walks ? kBwdBNLong : kBwdBN;
  // Their forward reads V transposed (a pre-pass writes V^T into the
  // workspace: plain 16-byte LDS reads instead of transposing ones; -5% on
  // one 75600-token document, the pre-pass included), for head dim 128 while
  // one head's V^T stays below 2 GiB.
  p.vt_pitch = vt_pitch_for(d.T);
  p.fwd_vt = long_walks && d.D == 128 && (int64_t)d.D * p.vt_pitch * 2 < ((int64_t)1 << 31);

  // Forward tiles, longest first (LPT order over the workgroup queue).
  std::vector<FwdTile> fwd;
  std::vector<int32_t> fwd_doc;
  for (const Segment& s : segs) {
    for (int64_t off = 0; off < s.len; off += p.fwd_rows) {
      FwdTile t{};
      t.m0 = (int32_t)(s.m0 + off);
      t.n = (int32_t)std::min<int64_t>(p.fwd_rows, s.len - off);
      t.g0 = (int32_t)(s.g0 + off);
      t.e = (int32_t)s.e;
      // keys of the tile's real rows [g0, rend): from the first row's band
      // start to the last row's band end (rows' bands ascend with g)
      const int64_t rend = std::min<int64_t>(t.g0 + t.n, s.e);
      t.ks0 = rend > t.g0 ? (int32_t)key_lo(p.band, s.a, t.g0) : (int32_t)s.a;
      t.ke0 = rend > t.g0 ? (int32_t)(key_hi(p.band, s.e, rend - 1) + 1) : (int32_t)s.a;
      fwd.push_back(t);
      fwd_doc.push_back(s.doc);
    }
  }
  p.fwd = split_walks(lpt_order(fwd, [](const FwdTile& t) { return fwd_cost(t); }), d.H,
                      p.fwd_rows, d.max_key_splits, &p.split_groups, &p.split_slots,
                      &p.split_tiles);

  // Backward tiles: per document, the keys its local real rows attend -- per
  // run of consecutive rows, from the first row's band start to the last
  // row's band end (causal: [a, g_max] for the whole document) -- merged.
  const std::vector<DocRows> docs = doc_rows(segs);
  std::vector<BwdTile> bwd;
  std::vector<std::pair<int64_t, int64_t>> touched;  // [r0, r1), ascending, disjoint
  for (const DocRows& dr : docs) {
    std::vector<std::pair<int64_t, int64_t>> ivs;
    for (const DocRows::Run& rn : dr.runs) {
      const int64_t x0 = key_lo(p.band, dr.a, rn.g0);
      const int64_t x1 = key_hi(p.band, dr.e, rn.g0 + rn.n - 1) + 1;
      if (!ivs.empty() && x0 <= ivs.back().second)
        ivs.back().second = std::max(ivs.back().second, x1);
      else
        ivs.push_back({x0, x1});
    }
    for (const auto& iv : ivs) {
      add_key_tiles(dr, p.band, p.bwd_keys, iv.first, iv.second, bwd);
      touched.push_back(iv);
    }
  }
  p.bwd = lpt_order(bwd, [](const BwdTile& t) { return (int64_t)t.m_hi - t.m_lo; });

  // Untouched key rows: the complement of the touched ranges in [0, T).
  std::sort(touched.begin(), touched.end());
  p.touched = 0;
  for (auto& tr : touched) p.touched += tr.second - tr.first;
  p.zero = untouched_ranges({{0, d.T}}, touched);

  // Rank-major K/V: the inverse of the all-ranks permutation. Rank r's local
  // row m sits at rank-major position r * n_local + m; under NO_LOAD_BALANCE
  // (or cp_size 1) that is global row order and no map is needed.
  const bool reordered = d.strategy == THDCP_DUAL_CHUNK_SWAP && d.cp_size > 1;
  p.kv_mapped = reordered && d.kv_layout == THDCP_KV_RANK_MAJOR;
  p.kv_row.clear();
  if (reordered && (p.kv_mapped || d.p2p)) {
    p.kv_row.assign(d.T, 0);
    for (int32_t r = 0; r < d.cp_size; ++r)
      for (const Segment& sg : build_segments(p, r))
        for (int64_t i = 0; i < sg.len; ++i)
          p.kv_row[sg.g0 + i] = (int32_t)(r * p.n_local + sg.m0 + i);
  }

  // P2P steps ([PAD] "Describe the bug": per-step metadata of the P2P path,
  // built here once per batch instead of by helper launches at every step).
  p.steps.clear();
  p.step_fwd.clear();
  p.step_bwd.clear();
  p.step_zero.clear();
  if (d.p2p) {
    for (int64_t src = 0; src < d.cp_size; ++src) {
      thdcp_plan::Step st{};
      // Forward: each query tile keeps the part of its causal key range that
      // rank src holds (empty ranges still list the tile: its rows get O = 0,
      // LSE = -inf for this step).
      std::vector<FwdTile> sf;
      for (size_t i = 0; i < fwd.size(); ++i) {
        FwdTile t = fwd[i];
        const int64_t klo = t.ks0, khi = t.ke0;
        t.ks0 = t.ke0 = t.ks1 = t.ke1 = 0;
        if (fwd_doc[i] >= 0 && khi > klo) {
          int64_t lo[2], hi[2];
          const int nr = key_ranges_of(p, fwd_doc[i], src, lo, hi);
          int slot = 0;
          for (int r = 0; r < nr; ++r) {
            const int64_t x0 = std::max(lo[r], klo), x1 = std::min(hi[r], khi);
            if (x1 <= x0) continue;
            (slot == 0 ? t.ks0 : t.ks1) = (int32_t)x0;
            (slot == 0 ? t.ke0 : t.ke1) = (int32_t)x1;
            ++slot;
          }
        }
        sf.push_back(t);
      }
      sf = lpt_order(sf, [](const FwdTile& t) { return fwd_cost(t); });
      st.fwd0 = (int32_t)p.step_fwd.size();
      st.n_fwd = (int32_t)sf.size();
      p.step_fwd.insert(p.step_fwd.end(), sf.begin(), sf.end());
      // Backward: key tiles over rank src's keys that local queries attend.
      std::vector<BwdTile> sb;
      std::vector<std::pair<int64_t, int64_t>> st_touched;
      for (const DocRows& dr : docs) {
        int64_t lo[2], hi[2];
        const int nr = key_ranges_of(p, dr.doc, src, lo, hi);
        for (int r = 0; r < nr; ++r) {
          const int64_t x0 = std::max(lo[r], dr.a), x1 = std::min(hi[r], dr.gmax + 1);
          if (x1 <= x0) continue;
          add_key_tiles(dr, p.band, p.bwd_keys, x0, x1, sb);
          st_touched.push_back({x0, x1});
        }
      }
      sb = lpt_order(sb, [](const BwdTile& t) { return (int64_t)t.m_hi - t.m_lo; });
      st.bwd0 = (int32_t)p.step_bwd.size();
      st.n_bwd = (int32_t)sb.size();
      p.step_bwd.insert(p.step_bwd.end(), sb.begin(), sb.end());
      // Rank src's rows (its local block, padding and tail included) that
      // no local query attends: zeroed only when there are any.
      std::vector<std::pair<int64_t, int64_t>> own;
      for (const Segment& sg : build_segments(p, src)) own.push_back({sg.g0, sg.g0 + sg.len});
      std::sort(own.begin(), own.end());
      std::sort(st_touched.begin(), st_touched.end());
      const std::vector<ZeroRange> sz = untouched_ranges(own, st_touched);
      st.zero0 = (int32_t)p.step_zero.size();
      st.n_zero = (int32_t)sz.size();
      st.untouched = sz.empty() ? 0 : sz.back().before + (sz.back().r1 - sz.back().r0);
      p.step_zero.insert(p.step_zero.end(), sz.begin(), sz.end());
      p.steps.push_back(st);
    }
  }

  // Host image of the device tables.
  p.off_fwd = 0;
  p.off_bwd = align256(p.off_fwd + p.fwd.size() * sizeof(FwdTile));
  p.off_zero = align256(p.off_bwd + p.bwd.size() * sizeof(BwdTile));
  p.off_kvrow = align256(p.off_zero + p.zero.size() * sizeof(ZeroRange));
  p.off_sfwd = align256(p.off_kvrow + p.kv_row.size() * sizeof(int32_t));
  p.off_sbwd = align256(p.off_sfwd + p.step_fwd.size() * sizeof(FwdTile));
  p.off_szero = align256(p.off_sbwd + p.step_bwd.size() * sizeof(BwdTile));
  p.off_cnt = align256(p.off_szero + p.step_zero.size() * sizeof(ZeroRange));
  p.off_part = align256(p.off_cnt + (size_t)p.split_groups * d.H * sizeof(int32_t));
  p.ws_bytes =
      p.off_part + (size_t)p.split_slots * d.H * kSplitFloats(d.D, p.fwd_rows) * sizeof(float);
  if (p.fwd_vt) {
    p.off_vt = align256(p.ws_bytes);
    p.ws_bytes = p.off_vt + (size_t)d.H * d.D * p.vt_pitch * sizeof(uint16_t);
  }
  if (p.ws_bytes == 0) p.ws_bytes = 256;
  // the image covers the tables and the split counters (zero), not the scratch
  p.blob.assign(std::max<size_t>(p.off_part, 256), 0);
  auto put = [&](size_t off, const void* src, size_t n) {
    if (n) memcpy(p.blob.data() + off, src, n);
  };
  put(p.off_fwd, p.fwd.data(), p.fwd.size() * sizeof(FwdTile));
  put(p.off_bwd, p.bwd.data(), p.bwd.size() * sizeof(BwdTile));
  put(p.off_zero, p.zero.data(), p.zero.size() * sizeof(ZeroRange));
  put(p.off_kvrow, p.kv_row.data(), p.kv_row.size() * sizeof(int32_t));
  put(p.off_sfwd, p.step_fwd.data(), p.step_fwd.size() * sizeof(FwdTile));
  put(p.off_sbwd, p.step_bwd.data(), p.step_bwd.size() * sizeof(BwdTile));
  put(p.off_szero, p.step_zero.data(), p.step_zero.size() * sizeof(ZeroRange));
}

// Counters and scratch of the all-gather tables' split key walks.
SplitWs split_ws(const thdcp_plan* p) {
  return {reinterpret_cast<int32_t*>(p->ws_dev + p->off_cnt),
          reinterpret_cast<float*>(p->ws_dev + p->off_part)};
}

// Row addressing of the all-gather calls' K/V (and dK/dV): rank-major
// through the map, or global order.
KvRows kv_map(const thdcp_plan* p) {
  return {p->kv_mapped ? reinterpret_cast<const int32_t*>(p->ws_dev + p->off_kvrow) : nullptr, 0,
          p->desc.T};
}

// Row addressing of a P2P step's K/V (and dK/dV): rank src's local block,
// n_local rows, in which global key g sits at row pos(g) - src * n_local.
KvRows kv_step(const thdcp_plan* p, int64_t src) {
  const bool mapped = !p->kv_row.empty();
  return {mapped ? reinterpret_cast<const int32_t*>(p->ws_dev + p->off_kvrow) : nullptr,
          src * p->n_local, p->n_local};
}

}  // namespace

extern "C" {

const char* thdcp_last_error(void) { return g_last_error.c_str(); }

int32_t thdcp_version(void) { return 100; }

thdcp_status_t thdcp_validate(const int32_t* cu_seqlens_host, const int32_t* cu_seqlens_padded_host,
                              int32_t B, int64_t T, int32_t cp_size, int32_t rank,
                              thdcp_strategy_t strategy, int32_t window_left,
                              int32_t window_right, int32_t pad_between_seqs,
                              int32_t* padding_present_out) {
  return check_layout(cu_seqlens_host, cu_seqlens_padded_host, B, T, cp_size, rank, strategy,
                      window_left, window_right, pad_between_seqs, padding_present_out);
}

thdcp_status_t thd_partition_index(const int32_t* cup_host, const int32_t* cup_dev, int32_t B,
                                   int64_t T, int32_t cp_size, int32_t rank,
                                   thdcp_strategy_t strategy, int32_t* idx_out_dev,
                                   void* stream) {
  if (!cup_dev || !idx_out_dev) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (cp_size < 1 || rank < -1 || rank >= cp_size)
    return fail(THDCP_ERR_ARG, "bad cp_size/rank (%d, %d)", cp_size, rank);
  if (B < 0 || T < 0 || T > INT32_MAX / 2) return fail(THDCP_ERR_ARG, "bad B or T");
  if (T % cp_size != 0) return fail(THDCP_ERR_LAYOUT, "T is not divisible by cp_size");
  if (strategy != THDCP_DUAL_CHUNK_SWAP && strategy != THDCP_NO_LOAD_BALANCE)
    return fail(THDCP_ERR_ARG, "unknown strategy %d", strategy);
  // Checked on every call (no host data needed): DUAL_CHUNK_SWAP cuts
  // documents into chunks, so rows with no document at all cannot be placed.
  if (strategy == THDCP_DUAL_CHUNK_SWAP && B == 0 && T > 0)
    return fail(THDCP_ERR_LAYOUT, "DUAL_CHUNK_SWAP with no documents needs T == 0 (got %lld)",
                (long long)T);
  if (cup_host) {
    thdcp_status_t st = check_layout(nullptr, cup_host, B, T, cp_size, rank < 0 ? 0 : rank,
                                     strategy, -1, 0, -1, nullptr);
    if (st != THDCP_OK) return st;
  }
  const int64_t n_out = rank < 0 ? T : T / cp_size;
  if (n_out == 0) return ok();
  return hip_status(launch_partition(cup_dev, B, T, cp_size, rank, strategy, idx_out_dev, n_out,
                                     (hipStream_t)stream),
                    "thd_partition_index launch");
}

thdcp_status_t thd_gather(const void* src, int64_t n_src, const int32_t* idx, int64_t n,
                          int64_t row_bytes, void* dst, void* stream) {
  return thd_gather_batched(1, &src, n_src, idx, n, row_bytes, &dst, stream);
}

thdcp_status_t thd_scatter(const void* src, int64_t n, const int32_t* idx, int64_t row_bytes,
                           void* dst, int64_t n_dst, void* stream) {
  return thd_scatter_batched(1, &src, n, idx, row_bytes, &dst, n_dst, stream);
}

namespace {
// Pointer lists are only checked when there is something to move: an empty
// move (no rows) succeeds whatever the pointers are.
thdcp_status_t check_count(int32_t n_tensors) {
  if (n_tensors < 1 || n_tensors > kMaxMoveTensors)
    return fail(THDCP_ERR_ARG, "n_tensors must be in [1, %d]", kMaxMoveTensors);
  return ok();
}

thdcp_status_t check_batch(int32_t n_tensors, const void* const* srcs, void* const* dsts) {
  if (check_count(n_tensors) != THDCP_OK) return THDCP_ERR_ARG;
  if (!srcs || !dsts) return fail(THDCP_ERR_ARG, "NULL pointer list");
  for (int32_t i = 0; i < n_tensors; ++i)
    if (!srcs[i] || !dsts[i]) return fail(THDCP_ERR_ARG, "NULL device pointer in list");
  return ok();
}
}  // namespace

thdcp_status_t thd_gather_batched(int32_t n_tensors, const void* const* srcs, int64_t n_src,
                                  const int32_t* idx, int64_t n, int64_t row_bytes,
                                  void* const* dsts, void* stream) {
  if (n < 0 || n_src < 0 || row_bytes <= 0) return fail(THDCP_ERR_ARG, "bad sizes");
  if (check_count(n_tensors) != THDCP_OK) return THDCP_ERR_ARG;
  if (n == 0) return ok();
  thdcp_status_t st = check_batch(n_tensors, srcs, dsts);
  if (st != THDCP_OK) return st;
  if (!idx) return fail(THDCP_ERR_ARG, "NULL index pointer");
  return hip_status(launch_gather(n_tensors, srcs, n_src, idx, n, row_bytes, dsts,
                                  (hipStream_t)stream),
                    "thd_gather launch");
}

thdcp_status_t thd_scatter_batched(int32_t n_tensors, const void* const* srcs, int64_t n,
                                   const int32_t* idx, int64_t row_bytes, void* const* dsts,
                                   int64_t n_dst, void* stream) {
  if (n < 0 || n_dst < 0 || row_bytes <= 0) return fail(THDCP_ERR_ARG, "bad sizes");
  if (check_count(n_tensors) != THDCP_OK) return THDCP_ERR_ARG;
  if (n == 0) return ok();
  thdcp_status_t st = check_batch(n_tensors, srcs, dsts);
  if (st != THDCP_OK) return st;
  if (!idx) return fail(THDCP_ERR_ARG, "NULL index pointer");
  return hip_status(launch_scatter(n_tensors, srcs, n, idx, row_bytes, dsts, n_dst,
                                   (hipStream_t)stream),
                    "thd_scatter launch");
}

namespace {
thdcp_status_t a2a_move(int32_t n_tensors, const void* const* srcs, int64_t n_tokens,
                        int32_t cp_size, int64_t group_bytes, void* const* dsts, bool unpack,
                        void* stream) {
  if (n_tokens < 0 || cp_size < 1 || group_bytes <= 0)
    return fail(THDCP_ERR_ARG, "bad sizes (n_tokens %lld, cp_size %d, group_bytes %lld)",
                (long long)n_tokens, cp_size, (long long)group_bytes);
  if (n_tokens * (int64_t)cp_size > INT32_MAX)
    return fail(THDCP_ERR_ARG, "n_tokens * cp_size exceeds int32");
  if (check_count(n_tensors) != THDCP_OK) return THDCP_ERR_ARG;
  if (n_tokens == 0) return ok();
  thdcp_status_t st = check_batch(n_tensors, srcs, dsts);
  if (st != THDCP_OK) return st;
  return hip_status(launch_a2a(n_tensors, srcs, n_tokens, cp_size, group_bytes, dsts, unpack,
                               (hipStream_t)stream),
                    unpack ? "thd_a2a_unpack launch" : "thd_a2a_pack launch");
}
}  // namespace

thdcp_status_t thd_a2a_pack(int32_t n_tensors, const void* const* srcs, int64_t n_tokens,
                            int32_t cp_size, int64_t group_bytes, void* const* dsts,
                            void* stream) {
  return a2a_move(n_tensors, srcs, n_tokens, cp_size, group_bytes, dsts, false, stream);
}

thdcp_status_t thd_a2a_unpack(int32_t n_tensors, const void* const* srcs, int64_t n_tokens,
                              int32_t cp_size, int64_t group_bytes, void* const* dsts,
                              void* stream) {
  return a2a_move(n_tensors, srcs, n_tokens, cp_size, group_bytes, dsts, true, stream);
}

thdcp_status_t thdcp_plan_create(const thdcp_attn_desc* desc, thdcp_plan_t* plan_out) {
  if (!desc || !plan_out) return fail(THDCP_ERR_ARG, "NULL argument");
  *plan_out = nullptr;
  const thdcp_attn_desc& d = *desc;
  if (d.H < 1) return fail(THDCP_ERR_ARG, "H must be >= 1");
  if (d.D != 64 && d.D != 128) return fail(THDCP_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d.D);
  int32_t padding = 0;
  thdcp_status_t st = check_layout(d.cu_seqlens_host, d.cu_seqlens_padded_host, d.B, d.T,
                                   d.cp_size, d.rank, d.strategy, d.window_left, d.window_right,
                                   d.pad_between_seqs, &padding);
  if (st != THDCP_OK) return st;
  const int64_t n_local = d.T / d.cp_size;
  if (n_local * (int64_t)d.H * d.D > ((int64_t)1 << 40)) return fail(THDCP_ERR_ARG, "too large");
  {
    // The attention kernels reach one document's K/V rows, and the local
    // Q/dO rows, through 32-bit buffer offsets; rows they skip use an offset
    // past every descriptor, so descriptors stay below 2 GiB.
    const int64_t row_bytes = (int64_t)d.H * d.D * 2;
    int64_t max_doc = 0;
    for (int32_t i = 0; i < d.B; ++i)
      max_doc = std::max<int64_t>(max_doc, (int64_t)d.cu_seqlens_padded_host[i + 1] -
                                               d.cu_seqlens_padded_host[i]);
    if (max_doc * row_bytes >= ((int64_t)1 << 31) || n_local * row_bytes >= ((int64_t)1 << 31))
      return fail(THDCP_ERR_UNSUPPORTED,
                  "a document (%lld rows) or the local share (%lld rows) exceeds 2 GiB of "
                  "bf16 rows of %lld bytes",
                  (long long)max_doc, (long long)n_local, (long long)row_bytes);
    if (d.kv_layout != THDCP_KV_GLOBAL && d.kv_layout != THDCP_KV_RANK_MAJOR)
      return fail(THDCP_ERR_ARG, "kv_layout %d (0 global, 1 rank-major)", d.kv_layout);
    if (d.p2p != 0 && d.p2p != 1) return fail(THDCP_ERR_ARG, "p2p %d (0 or 1)", d.p2p);
    if (d.max_key_splits < 0)
      return fail(THDCP_ERR_ARG, "max_key_splits %d (0 automatic, 1 never, n at most n)",
                  d.max_key_splits);
    if (d.p2p && (d.window_left != -1 || d.window_right != 0))
      return fail(THDCP_ERR_UNSUPPORTED,
                  "P2P steps take the causal mask only, window_size=(-1, 0) (got (%d, %d))",
                  d.window_left, d.window_right);
    // Mapped K/V rows are addressed from the start of the buffer.
    if (d.kv_layout == THDCP_KV_RANK_MAJOR && d.T * row_bytes >= ((int64_t)1 << 31))
      return fail(THDCP_ERR_UNSUPPORTED,
                  "rank-major K/V of %lld rows exceeds 2 GiB of bf16 rows of %lld bytes",
                  (long long)d.T, (long long)row_bytes);
  }
  thdcp_plan* p = new (std::nothrow) thdcp_plan();
  if (!p) return fail(THDCP_ERR_ARG, "out of host memory");
  p->desc = d;
  p->cup.assign(d.cu_seqlens_padded_host, d.cu_seqlens_padded_host + d.B + 1);
  if (d.cu_seqlens_host)
    p->cu.assign(d.cu_seqlens_host, d.cu_seqlens_host + d.B + 1);
  else
    p->cu = p->cup;
  p->desc.cu_seqlens_host = nullptr;  // the plan keeps its own copies
  p->desc.cu_seqlens_padded_host = nullptr;
  p->n_local = n_local;
  p->scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.0f / std::sqrt((float)d.D);
  p->padding = padding;
  // A side at or past T is no bound (T < 2^30, so kUnbounded covers it).
  const int32_t wl = (d.window_left < 0 || d.window_left >= d.T) ? kUnbounded : d.window_left;
  const int32_t wr = (d.window_right < 0 || d.window_right >= d.T) ? kUnbounded : d.window_right;
  p->band = Band{wl, wr, wl == kUnbounded && wr == 0};
  build_plan(*p);
  *plan_out = p;
  return ok();
}

thdcp_status_t thdcp_plan_get_info(thdcp_plan_t p, thdcp_plan_info* info) {
  if (!p || !info) return fail(THDCP_ERR_ARG, "NULL argument");
  info->n_local = p->n_local;
  info->causal_pairs = p->pairs;
  info->touched_rows = p->touched;
  info->untouched_rows = p->desc.T - p->touched;
  info->padding_present = p->padding;
  info->n_fwd_tiles = 0;
  for (const FwdTile& t : p->fwd) info->n_fwd_tiles += t.part == 0;
  info->n_bwd_tiles = (int32_t)p->bwd.size();
  info->n_zero_ranges = (int32_t)p->zero.size();
  info->workspace_bytes = p->ws_bytes;
  info->bwd_scratch_bytes = align256((size_t)p->n_local * p->desc.H * sizeof(float));
  info->n_split_tiles = p->split_tiles;
  info->n_fwd_parts = (int32_t)p->fwd.size();
  info->fwd_tile_rows = p->fwd_rows;
  info->bwd_tile_keys = p->bwd_keys;
  return ok();
}

thdcp_status_t thdcp_plan_local_seqlens(thdcp_plan_t p, int32_t* out) {
  if (!p || !out) return fail(THDCP_ERR_ARG, "NULL argument");
  std::copy(p->local_seqlens.begin(), p->local_seqlens.end(), out);
  return ok();
}

namespace {

// Page-locked staging for plan uploads. An asynchronous host-to-device copy
// inside the compute stream (pageable or page-locked source) left 15-30 us of
// idle GPU time per upload on MI355X, the largest gap in a dcs_8k step. The
// plan is instead copied into a page-locked slot on the host and moved into
// the workspace by a small copy kernel on the same stream, which reads the
// slot over the host link. Slots live until the process exits (never freed
// while a copy may read them). Each upload takes a slot whose last copy has
// finished, found with non-blocking event queries; when every slot is still
// in use (the host is that many uploads ahead of the GPU) a new block of
// slots is allocated, up to kMaxSlots. Only past that does an upload wait for
// the oldest slot's copy.
class StagingRing {
 public:
  static constexpr size_t kSlotBytes = size_t(1) << 20;
  static constexpr int kBlockSlots = 16;
  static constexpr int kMaxSlots = 64;

  // Enqueues the copy of n bytes at src to dst on stream. Returns false (and
  // enqueues nothing) when the ring cannot take it: n above a slot, or the
  // first page-locked allocation failed; the caller then copies directly.
  bool upload(void* dst, const void* src, size_t n, hipStream_t stream, hipError_t* err) {
    if (n > kSlotBytes) return false;
    std::lock_guard<std::mutex> lock(mu_);
    if (slots_.empty() && !grow()) return false;
    Slot* sl = nullptr;
    const size_t count = slots_.size();
    for (size_t i = 0; i < count && !sl; ++i) {  // round robin from the last used slot
      Slot& c = slots_[(next_ + i) % count];
      if (c.pending) {
        const hipError_t q = hipEventQuery(c.ev);
        if (q == hipErrorNotReady) continue;
        if (q != hipSuccess) {
          *err = q;
          return true;
        }
        c.pending = false;
      }
      sl = &c;
      next_ = (next_ + i + 1) % count;
    }
    if (!sl && count < (size_t)kMaxSlots && grow()) {
      sl = &slots_[count];  // the first slot of the new block
      next_ = (count + 1) % slots_.size();
    }
    if (!sl) {  // kMaxSlots copies in flight: wait for the oldest
      sl = &slots_[next_];
      next_ = (next_ + 1) % count;
      *err = hipEventSynchronize(sl->ev);
      if (*err != hipSuccess) return true;
      sl->pending = false;
    }
    memcpy(sl->host, src, n);
    *err = launch_copy16(sl->dev, dst, (int64_t)n, stream);
    if (*err != hipSuccess) return true;
    *err = hipEventRecord(sl->ev, stream);
    sl->pending = *err == hipSuccess;
    return true;
  }

  size_t slots() {
    std::lock_guard<std::mutex> lock(mu_);
    return slots_.size();
  }

 private:
  struct Slot {
    char* host = nullptr;
    const void* dev = nullptr;  // the slot as the GPU addresses it
    hipEvent_t ev = nullptr;
    bool pending = false;
  };

  // One more block of kBlockSlots slots; false (and the ring unchanged) if
  // an allocation fails. A block that fails half way stays allocated.
  bool grow() {
    if (failed_) return false;
    char* base = nullptr;
    if (hipHostMalloc(reinterpret_cast<void**>(&base), kSlotBytes * kBlockSlots,
                      hipHostMallocPortable | hipHostMallocMapped) != hipSuccess) {
      failed_ = slots_.empty();
      return false;
    }
    void* dbase = nullptr;
    if (hipHostGetDevicePointer(&dbase, base, 0) != hipSuccess) {
      failed_ = slots_.empty();
      return false;
    }
    std::vector<Slot> block(kBlockSlots);
    for (int i = 0; i < kBlockSlots; ++i) {
      block[i].host = base + i * kSlotBytes;
      block[i].dev = static_cast<const char*>(dbase) + i * kSlotBytes;
      if (hipEventCreateWithFlags(&block[i].ev, hipEventDisableTiming) != hipSuccess) {
        failed_ = slots_.empty();
        return false;
      }
    }
    slots_.insert(slots_.end(), block.begin(), block.end());
    return true;
  }

  std::mutex mu_;
  std::vector<Slot> slots_;
  size_t next_ = 0;
  bool failed_ = false;
};

StagingRing& staging_ring() {
  static StagingRing* ring = new StagingRing();  // never destroyed: copies may be in flight at exit
  return *ring;
}

}  // namespace

thdcp_status_t thdcp_plan_upload(thdcp_plan_t p, void* ws, size_t bytes, void* stream) {
  if (!p || !ws) return fail(THDCP_ERR_ARG, "NULL argument");
  if (bytes < p->ws_bytes)
    return fail(THDCP_ERR_ARG, "workspace of %zu bytes is below the %zu the plan needs", bytes,
                p->ws_bytes);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(THDCP_ERR_ARG, "workspace must be 256-byte aligned");
  hipError_t e = hipSuccess;
  if (!staging_ring().upload(ws, p->blob.data(), p->blob.size(), (hipStream_t)stream, &e))
    e = hipMemcpyAsync(ws, p->blob.data(), p->blob.size(), hipMemcpyHostToDevice,
                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "plan upload");
  p->ws_dev = static_cast<char*>(ws);
  return ok();
}

void thdcp_plan_destroy(thdcp_plan_t p) { delete p; }

thdcp_status_t cp_attn_fwd(thdcp_plan_t p, const void* q, const void* k, const void* v, void* o,
                           float* lse, void* stream) {
  if (!p) return fail(THDCP_ERR_ARG, "NULL plan");
  if (!p->ws_dev) return fail(THDCP_ERR_ARG, "plan not uploaded (call thdcp_plan_upload)");
  if (p->n_local == 0) return ok();
  if (!q || !k || !v || !o || !lse) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(THDCP_ERR_ARG, "Q/K/V/O must be 16-byte aligned");
  if (p->fwd.empty()) return ok();
  void* vt = nullptr;
  if (p->fwd_vt) {
    vt = p->ws_dev + p->off_vt;
    hipError_t e = launch_v_transpose(v, kv_map(p), p->desc.H, p->desc.D,
                                      reinterpret_cast<const ZeroRange*>(p->ws_dev + p->off_zero),
                                      (int32_t)p->zero.size(), vt, p->vt_pitch, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "cp_attn_fwd transpose launch");
  }
  return hip_status(
      launch_attn_fwd(reinterpret_cast<const FwdTile*>(p->ws_dev + p->off_fwd),
                      (int32_t)p->fwd.size(), p->desc.H, p->desc.D, p->fwd_rows, q, k, v,
                      kv_map(p), p->band, o, lse, p->n_local, p->scale, split_ws(p), vt,
                      p->vt_pitch, (hipStream_t)stream),
      "cp_attn_fwd launch");
}

namespace {

thdcp_status_t check_plan(thdcp_plan_t p) {
  if (!p) return fail(THDCP_ERR_ARG, "NULL plan");
  if (!p->ws_dev) return fail(THDCP_ERR_ARG, "plan not uploaded (call thdcp_plan_upload)");
  return ok();
}

size_t scratch_need(thdcp_plan_t p) {
  return align256((size_t)p->n_local * p->desc.H * sizeof(float));
}

}  // namespace

thdcp_status_t cp_attn_bwd_preprocess(thdcp_plan_t p, const void* o, const float* lse,
                                      const void* d_o, void* scratch, size_t scratch_bytes,
                                      void* stream) {
  thdcp_status_t st = check_plan(p);
  if (st != THDCP_OK) return st;
  if (!o || !lse || !d_o) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(o) || !aligned16(d_o)) return fail(THDCP_ERR_ARG, "O/dO must be 16-byte aligned");
  if (!scratch || scratch_bytes < scratch_need(p))
    return fail(THDCP_ERR_ARG, "scratch of %zu bytes is below the %zu needed", scratch_bytes,
                scratch_need(p));
  if (p->n_local == 0) return ok();
  return hip_status(launch_bwd_prep(o, d_o, lse, static_cast<float*>(scratch), p->n_local,
                                    p->desc.H, p->desc.D, (hipStream_t)stream),
                    "cp_attn_bwd_preprocess launch");
}

namespace {

thdcp_status_t check_bwd_inputs(thdcp_plan_t p, const void* q, const void* k, const void* v,
                                const float* lse, const void* d_o, const void* scratch,
                                size_t scratch_bytes) {
  if (!q || !k || !v || !lse || !d_o) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o))
    return fail(THDCP_ERR_ARG, "tensors must be 16-byte aligned");
  if (!scratch || scratch_bytes < scratch_need(p))
    return fail(THDCP_ERR_ARG, "scratch of %zu bytes is below the %zu needed", scratch_bytes,
                scratch_need(p));
  return ok();
}

}  // namespace

thdcp_status_t cp_attn_bwd_dkdv(thdcp_plan_t p, const void* q, const void* k, const void* v,
                                const float* lse, const void* d_o, float* dk, float* dv,
                                int32_t accumulate_dkv, const void* scratch, size_t scratch_bytes,
                                void* stream) {
  thdcp_status_t st = check_plan(p);
  if (st != THDCP_OK) return st;
  st = check_bwd_inputs(p, q, k, v, lse, d_o, scratch, scratch_bytes);
  if (st != THDCP_OK) return st;
  if (!dk || !dv) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(dk) || !aligned16(dv)) return fail(THDCP_ERR_ARG, "dK/dV must be 16-byte aligned");
  if (p->bwd.empty()) return ok();
  return hip_status(
      launch_attn_bwd_dkdv(reinterpret_cast<const BwdTile*>(p->ws_dev + p->off_bwd),
                           (int32_t)p->bwd.size(), p->desc.H, p->desc.D, p->bwd_keys, q, k, v,
                           kv_map(p), p->band,
                           d_o, lse, static_cast<const float*>(scratch), dk, dv, p->n_local,
                           p->scale, accumulate_dkv, (hipStream_t)stream),
      "cp_attn_bwd_dkdv launch");
}

thdcp_status_t cp_attn_bwd_dq(thdcp_plan_t p, const void* q, const void* k, const void* v,
                              const float* lse, const void* d_o, float* dq, const void* scratch,
                              size_t scratch_bytes, void* stream) {
  thdcp_status_t st = check_plan(p);
  if (st != THDCP_OK) return st;
  st = check_bwd_inputs(p, q, k, v, lse, d_o, scratch, scratch_bytes);
  if (st != THDCP_OK) return st;
  if (!dq) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(dq)) return fail(THDCP_ERR_ARG, "dQ must be 16-byte aligned");
  if (p->fwd.empty()) return ok();
  return hip_status(
      launch_attn_bwd_dq(reinterpret_cast<const FwdTile*>(p->ws_dev + p->off_fwd),
                         (int32_t)p->fwd.size(), p->desc.H, p->desc.D, p->fwd_rows, q, k, v,
                         kv_map(p), p->band, d_o,
                         nullptr, lse, static_cast<float*>(const_cast<void*>(scratch)), dq,
                         p->n_local, p->scale, 0, split_ws(p), DqExtras{}, (hipStream_t)stream),
      "cp_attn_bwd_dq launch");
}

thdcp_status_t thdcp_lse_merge_parts(int64_t n, int32_t H, int32_t D, int32_t parts,
                                     const void* o_parts, const float* lse_parts, void* o_out,
                                     float* lse_out, void* stream) {
  if (n < 0 || H < 1 || parts < 1) return fail(THDCP_ERR_ARG, "bad size");
  if (D != 64 && D != 128) return fail(THDCP_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (n == 0) return ok();
  if (!o_parts || !lse_parts || !o_out) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(o_parts) || !aligned16(o_out))
    return fail(THDCP_ERR_ARG, "O buffers must be 16-byte aligned");
  return hip_status(launch_lse_merge_parts(n, H, D, parts, o_parts, lse_parts, o_out, lse_out,
                                           (hipStream_t)stream),
                    "thdcp_lse_merge_parts launch");
}

thdcp_status_t thdcp_zero_untouched(thdcp_plan_t p, float* dk, float* dv, void* stream) {
  thdcp_status_t st = check_plan(p);
  if (st != THDCP_OK) return st;
  if (!dk || !dv) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(dk) || !aligned16(dv)) return fail(THDCP_ERR_ARG, "dK/dV must be 16-byte aligned");
  // Gated: nothing is enqueued when every key row is attended by some local query.
  if (p->zero.empty()) return ok();
  const int64_t rows = p->desc.T - p->touched;
  return hip_status(launch_zero_rows(reinterpret_cast<const ZeroRange*>(p->ws_dev + p->off_zero),
                                     (int32_t)p->zero.size(), rows, kv_map(p),
                                     (int64_t)p->desc.H * p->desc.D, dk, dv, (hipStream_t)stream),
                    "thdcp_zero_untouched launch");
}

thdcp_status_t cp_attn_bwd(thdcp_plan_t p, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* d_o, float* dq,
                           float* dk, float* dv, int32_t zero_untouched, int32_t accumulate_dkv,
                           void* scratch, size_t scratch_bytes, void* stream) {
  thdcp_status_t st = check_plan(p);
  if (st != THDCP_OK) return st;
  if (zero_untouched && accumulate_dkv)
    return fail(THDCP_ERR_ARG, "zero_untouched and accumulate_dkv are mutually exclusive");
  if (!o) return fail(THDCP_ERR_ARG, "NULL device pointer");
  // Check every argument before enqueuing anything.
  if (!q || !k || !v || !lse || !d_o || !dq || !dk || !dv)
    return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(THDCP_ERR_ARG, "tensors must be 16-byte aligned");
  if (!scratch || scratch_bytes < scratch_need(p))
    return fail(THDCP_ERR_ARG, "scratch of %zu bytes is below the %zu needed", scratch_bytes,
                scratch_need(p));
  if (p->n_local == 0) {
    if (zero_untouched) return thdcp_zero_untouched(p, dk, dv, stream);
    return ok();
  }
  // Two launches. The dQ kernel also computes delta = rowsum(dO * O) into the
  // scratch (no separate preprocess launch), and its grid ends with the gated
  // zeroing of untouched dK/dV rows when the caller asks for it and the plan
  // has such rows (no separate zeroing launch). Then the dK/dV kernel.
  float* delta = static_cast<float*>(scratch);
  DqExtras ex;
  if (zero_untouched && !p->zero.empty()) {
    ex.zr = reinterpret_cast<const ZeroRange*>(p->ws_dev + p->off_zero);
    ex.n_zr = (int32_t)p->zero.size();
    ex.zero_rows = p->desc.T - p->touched;
    ex.dk = dk;
    ex.dv = dv;
  }
  {
    hipError_t e = launch_attn_bwd_dq(reinterpret_cast<const FwdTile*>(p->ws_dev + p->off_fwd),
                                      (int32_t)p->fwd.size(), p->desc.H, p->desc.D,
                                      p->fwd_rows, q, k, v, kv_map(p), p->band, d_o, o, lse, delta, dq, p->n_local,
                                      p->scale, 0, split_ws(p), ex, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "cp_attn_bwd dq launch");
  }
  if (!p->bwd.empty()) {
    hipError_t e = launch_attn_bwd_dkdv(
        reinterpret_cast<const BwdTile*>(p->ws_dev + p->off_bwd), (int32_t)p->bwd.size(),
        p->desc.H, p->desc.D, p->bwd_keys, q, k, v, kv_map(p), p->band, d_o, lse, delta, dk, dv,
        p->n_local,
        p->scale, accumulate_dkv, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "cp_attn_bwd dkdv launch");
  }
  return ok();
}

// ---------------------------------------------------------------------------
// P2P (ring) steps
// ---------------------------------------------------------------------------
namespace {

thdcp_status_t check_step(thdcp_plan_t p, int32_t src) {
  thdcp_status_t st = check_plan(p);
  if (st != THDCP_OK) return st;
  if (!p->desc.p2p) return fail(THDCP_ERR_ARG, "the plan was not made with p2p = 1");
  if (src < 0 || src >= p->desc.cp_size)
    return fail(THDCP_ERR_ARG, "src_rank %d outside [0, %d)", src, p->desc.cp_size);
  return ok();
}

}  // namespace

thdcp_status_t cp_attn_fwd_step(thdcp_plan_t p, int32_t src, const void* q, const void* k,
                                const void* v, void* o, float* lse, void* stream) {
  thdcp_status_t st = check_step(p, src);
  if (st != THDCP_OK) return st;
  if (p->n_local == 0) return ok();
  if (!q || !k || !v || !o || !lse) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(THDCP_ERR_ARG, "Q/K/V/O must be 16-byte aligned");
  const thdcp_plan::Step& sp = p->steps[src];
  if (sp.n_fwd == 0) return ok();
  return hip_status(
      launch_attn_fwd(reinterpret_cast<const FwdTile*>(p->ws_dev + p->off_sfwd) + sp.fwd0,
                      sp.n_fwd, p->desc.H, p->desc.D, p->fwd_rows, q, k, v, kv_step(p, src),
                      p->band, o, lse, p->n_local, p->scale, SplitWs{}, nullptr, 0,
                      (hipStream_t)stream),
      "cp_attn_fwd_step launch");
}

thdcp_status_t thdcp_lse_merge(int64_t n, int32_t H, int32_t D, const void* o_part,
                               const float* lse_part, float* o_acc, float* lse_acc,
                               int32_t first, void* o_out, void* stream) {
  if (n < 0 || H < 1) return fail(THDCP_ERR_ARG, "bad size");
  if (D != 64 && D != 128) return fail(THDCP_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", D);
  if (n == 0) return ok();
  if (!o_part || !lse_part || !o_acc || !lse_acc) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(o_part) || !aligned16(o_acc) || (o_out && !aligned16(o_out)))
    return fail(THDCP_ERR_ARG, "O buffers must be 16-byte aligned");
  return hip_status(launch_lse_merge(n, H, D, o_part, lse_part, o_acc, lse_acc, first != 0,
                                     o_out, (hipStream_t)stream),
                    "thdcp_lse_merge launch");
}

thdcp_status_t cp_attn_bwd_step(thdcp_plan_t p, int32_t src, const void* q, const void* k,
                                const void* v, const float* lse, const void* d_o,
                                const void* scratch, size_t scratch_bytes, float* dq,
                                int32_t accumulate_dq, float* dk, float* dv,
                                int32_t zero_untouched, void* stream) {
  thdcp_status_t st = check_step(p, src);
  if (st != THDCP_OK) return st;
  st = check_bwd_inputs(p, q, k, v, lse, d_o, scratch, scratch_bytes);
  if (st != THDCP_OK) return st;
  if (!dq || !dk || !dv) return fail(THDCP_ERR_ARG, "NULL device pointer");
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(THDCP_ERR_ARG, "dQ/dK/dV must be 16-byte aligned");
  if (p->n_local == 0) return ok();
  const thdcp_plan::Step& sp = p->steps[src];
  const KvRows kv = kv_step(p, src);
  float* delta = static_cast<float*>(const_cast<void*>(scratch));
  // The dQ launch also zeroes the peer's rows no local query reaches, with
  // workgroups at the end of its grid, when there are any.
  DqExtras ex;
  if (zero_untouched && sp.n_zero > 0) {
    ex.zr = reinterpret_cast<const ZeroRange*>(p->ws_dev + p->off_szero) + sp.zero0;
    ex.n_zr = sp.n_zero;
    ex.zero_rows = sp.untouched;
    ex.dk = dk;
    ex.dv = dv;
  }
  if (sp.n_fwd > 0 || ex.zr) {
    hipError_t e = launch_attn_bwd_dq(
        reinterpret_cast<const FwdTile*>(p->ws_dev + p->off_sfwd) + sp.fwd0, sp.n_fwd,
        p->desc.H, p->desc.D, p->fwd_rows, q, k, v, kv, p->band, d_o, nullptr, lse, delta, dq,
        p->n_local,
        p->scale, accumulate_dq != 0, SplitWs{}, ex, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "cp_attn_bwd_step dq launch");
  }
  if (sp.n_bwd > 0) {
    hipError_t e = launch_attn_bwd_dkdv(
        reinterpret_cast<const BwdTile*>(p->ws_dev + p->off_sbwd) + sp.bwd0, sp.n_bwd, p->desc.H,
        p->desc.D, p->bwd_keys, q, k, v, kv, p->band, d_o, lse, delta, dk, dv, p->n_local,
        p->scale, 0,
        (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "cp_attn_bwd_step dkdv launch");
  }
  return ok();
}

}  // extern "C"
