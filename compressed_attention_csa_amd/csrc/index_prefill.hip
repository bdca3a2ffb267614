// Lightning-Indexer scoring with streaming exact top-k for many query tokens (prefill).
//
// V4 report digest, sections 三 and 七: every query token scores all visible
// compressed entries with the indexer and keeps the top-k; in a long prefill the
// full score matrix (queries x entries) is far too large to materialise, so the
// selection is fused into the scoring sweep.
//
// Work split.  A workgroup owns 32 query tokens of one sequence, 4 per wave over
// 8 waves (two waves per SIMD, so one wave's matrix products overlap the other
// wave's vector epilogue), and sweeps every entry visible to any of them.  Entry
// keys are staged in LDS in tiles of 256 entries (16-byte chunks XOR-swizzled by
// entry so the operand reads are conflict-free), double-buffered: while a tile
// is scored, the next one is already in LDS and the one after is in flight in
// registers.  All workgroups sweep the entries in the same order, so the
// workgroups of one XCD mostly hit its L2 for the shared keys.
//
// MFMA layout.  16x16x32 bf16 products with entries as columns.  A wave's 4
// queries fill a tile pair: tile A holds heads 0-3 and tile B heads 4-7 of the
// same 4 queries (row 4*q + h), so lane (g, col) receives all 8 head dots of
// query g for entry col and forms sum_h w_h * ReLU(dot_h) without any
// cross-lane exchange.  The products of the next 16 entries are issued before
// the current ones are reduced.  With e4m3 keys, either the codes are widened
// to bf16 when staged (bf16 products), or, in the fp8 x fp8 variant, they stay
// 8-bit in LDS and the query rows are quantised to e4m3 once per workgroup;
// then 16x16x32 fp8 products take the same lane layout, one 16-byte LDS read
// per lane holding both k-steps of a 64-dim key.
//
// Exact top-k.  Each query keeps a candidate buffer in the workspace and a
// threshold tau (a 64-bit rank key: score, then lower index first).  A binary32
// compare against tau's score screens every pair; the pairs that pass it are
// appended as (score, entry | query << 30), in entry order, to one LDS staging
// area per wave shared by its 4 queries: the compare is the write mask and the
// slot is the running count plus the lane's rank in the mask (so the scoring
// loop issues no global stores, whose pending completion would otherwise make
// every wait also drain the key prefetch).  Rank keys are formed, and tested
// exactly against their query's tau, when the staging area is drained to the
// query buffers, between tiles once it cannot take another tile.  When a
// buffer cannot take its query's staged pairs, a histogram pass over the keys
// relative to tau (bins spanning tau .. the largest key appended) and, if
// needed, finer radix passes raise tau to a bin edge that keeps between k and
// 5k/4 candidates, and the buffer is compacted in order.  Everything dropped
// ranks below at least k candidates already kept, so the final exact selection
// over the buffer is the exact top-k; the output lists the winners by
// increasing entry index.
#include <type_traits>

#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kWaves = kPrefillWaves;
constexpr int kThreads = kWaves * kWave;
constexpr int kTileE = 256;  // entries per LDS tile
constexpr int kHBits = 9;    // histogram digit
constexpr int kHBins = 1 << kHBits;
constexpr int kBatch = 8;    // buffer keys per lane per batch of loads
constexpr int kStage = kPrefillStage;  // LDS staging slots per wave
constexpr uint32_t kTagShift = 30;          // staged entry: index | query << 30

struct LdsPrefill {
  uint4 tile[2][kTileE * 8];  // up to 128 B per entry, two buffers
  float scale[2][kTileE];
  uint32_t hist[kWaves][kHBins];
  uint64_t stg[kWaves][kStage];  // appended (score, entry) pairs not yet in the workspace
};

// LDS position (in 16-byte chunks) of chunk c of entry e, for cpe = 4 or 8
// chunks per entry.  The chunk index is XORed with a function of the entry so
// that 8 lanes reading one chunk of 8 consecutive entries, 16 lanes reading
// one chunk of 16 consecutive entries, and 8 or 16 lanes writing consecutive
// chunks all hit distinct 16-byte bank groups.
__device__ __forceinline__ int chunk_pos(int e, int c, int cpe) {
  const int h = cpe == 8 ? ((e & 7) ^ ((e >> 3) & 1)) : (((e >> 1) & 3) ^ ((e >> 3) & 1));
  return e * cpe + (c ^ h);
}


__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = __shfl(uint32_t(v), src), hi = __shfl(uint32_t(v >> 32), src);
  return (uint64_t(hi) << 32) | lo;
}

// ---------------------------------------------------------------- wave-local selection
//
// buf holds n rank keys of one query, written by this wave; the caller has
// waited for its own stores to complete.

// Histogram (in hist[0 .. kHBins)) of digit(v) over the keys of buf[0..n) with
// v & mask == prefix; digit() must return a value below kHBins for those keys.
template <typename Digit>
__device__ void wave_hist(const uint64_t* buf, int n, uint64_t mask, uint64_t prefix, uint32_t* hist,
                          Digit digit) {
  const int lane = threadIdx.x & 63;
  for (int x = lane; x < kHBins; x += kWave) hist[x] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int x0 = 0; x0 < n; x0 += kWave * kBatch) {
    uint64_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int x = x0 + u * kWave + lane;
      v[u] = x < n ? buf[x] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int x = x0 + u * kWave + lane;
      if (x < n && (v[u] & mask) == prefix) atomicAdd(&hist[digit(v[u]) & (kHBins - 1)], 1u);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Over bins [0, nb) taken from the top: the bin d where the count from the top
// first reaches need; above = keys in bins above d, indig = keys in bin d.
__device__ void wave_find(const uint32_t* hist, uint32_t nb, int need, uint32_t& dstar, uint32_t& above,
                          uint32_t& indig) {
  const int lane = threadIdx.x & 63;
  const uint32_t bpl = nb >= kWave ? nb / kWave : 1u;  // bins per lane, descending
  uint32_t local = 0;
  if (uint32_t(lane) * bpl < nb)
    for (uint32_t j = 0; j < bpl; ++j) local += hist[nb - 1 - (lane * bpl + j)];
  uint32_t inc = local;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  const uint32_t ex = inc - local;
  uint32_t d = 0, ab = 0, in = 0;
  bool mine = false;
  if (uint32_t(lane) * bpl < nb && int(ex) < need && int(inc) >= need) {
    uint32_t cum = ex;
    for (uint32_t j = 0; j < bpl; ++j) {
      const uint32_t dd = nb - 1 - (lane * bpl + j);
      const uint32_t h = hist[dd];
      if (int(cum + h) >= need) {
        d = dd;
        ab = cum;
        in = h;
        break;
      }
      cum += h;
    }
    mine = true;
  }
  const uint64_t who = __ballot(mine);
  const int src = __ffsll((long long)who) - 1;
  dstar = __shfl(d, src);
  above = __shfl(ab, src);
  indig = __shfl(in, src);
  __builtin_amdgcn_wave_barrier();
}

// Threshold T over the n keys of buf (1 <= need <= n) with kept = #(keys >= T)
// >= need: exactly need if `exact`, else at most max(need, keep_max).  Every
// key is > floor_key and has its upper half <= top_hi.  The first pass bins the
// upper halves between floor_key's and top_hi; later passes refine 11 bits at
// a time inside the bin that holds the need-th key.
__device__ uint64_t wave_threshold(const uint64_t* buf, int n, int need, bool exact, int keep_max,
                                   uint64_t floor_key, uint32_t top_hi, uint32_t* hist, int& kept) {
  const uint32_t lo_hi = uint32_t(floor_key >> 32);
  int sh = 0;
  while ((top_hi >> sh) - (lo_hi >> sh) >= uint32_t(kHBins)) ++sh;
  const uint32_t base = lo_hi >> sh;
  wave_hist(buf, n, 0ull, 0ull, hist, [&](uint64_t v) { return int((uint32_t(v >> 32) >> sh) - base); });
  uint32_t d, above, indig;
  wave_find(hist, uint32_t(kHBins), need, d, above, indig);
  int hi_bit = 32 + sh;
  uint64_t prefix = uint64_t(base + d) << hi_bit;
  need -= int(above);
  int above_total = int(above);
  kept = above_total + int(indig);
  if (int(indig) == need || (!exact && kept <= keep_max)) return prefix;
  while (hi_bit > 0) {
    const int width = hi_bit >= kHBits ? kHBits : hi_bit;
    const int shift = hi_bit - width;
    const uint64_t mask = hi_bit >= 64 ? 0ull : (~0ull << hi_bit);
    wave_hist(buf, n, mask, prefix, hist, [&](uint64_t v) { return int(uint32_t(v >> shift) & ((1u << width) - 1u)); });
    wave_find(hist, 1u << width, need, d, above, indig);
    prefix |= uint64_t(d) << shift;
    need -= int(above);
    above_total += int(above);
    hi_bit = shift;
    kept = above_total + int(indig);
    if (int(indig) == need || (!exact && kept <= keep_max)) break;
  }
  return prefix;
}

// Keep the keys >= T of buf[0..n) in order (in place); returns the new count.
// Each batch is loaded whole before any of its keys is written back, and the
// write position never passes the read position.
__device__ int wave_compact(uint64_t* buf, int n, uint64_t T) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int out = 0;
  for (int x0 = 0; x0 < n; x0 += kWave * kBatch) {
    uint64_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int x = x0 + u * kWave + lane;
      v[u] = x < n ? buf[x] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int x = x0 + u * kWave + lane;
      const bool keep = x < n && v[u] >= T;
      const uint64_t m = __ballot(keep);
      if (keep) buf[out + __popcll(m & below)] = v[u];
      out += __popcll(m);
    }
  }
  return out;
}

// ---------------------------------------------------------------- kernel

// FH: all 8 head rows of the products are real heads (H_I == 8).  Otherwise
// the zero rows past H_I are left out of the head sum (0 times an infinite key
// element is NaN, which a zero weight would not remove).
// KK == kKeyE4M3Q8: the query rows are quantised to e4m3 on load and the
// products are fp8 x fp8 MFMAs on the raw key codes, which stay 8-bit in LDS.
// BS: the approximate selector (scores rounded to bf16), a template argument so
// that the exact selector's inner loop carries no rounding instructions.
template <int KK, int DI, bool FH, bool BS>
__global__ __launch_bounds__(kThreads) void idx_prefill_kernel(IndexArgs a, IndexPlan p) {
  __shared__ LdsPrefill L;
  debug_poison_lds(L);
  constexpr bool Q8 = KK == kKeyE4M3Q8;
  constexpr int KB = key_is_e4m3(KK) ? 1 : 2;  // key bytes per element
  constexpr int CPG = DI * KB / 16;              // 16-byte chunks per entry in memory
  constexpr int CPE = Q8 ? CPG : DI / 8;         // 16-byte chunks per entry in LDS (bf16, or raw codes)
  constexpr int KSTEP = DI / 32;                 // 32-wide k-steps of one dot product
  constexpr int TE = kTileE;                      // entries per tile
  constexpr int CHUNKS = TE * CPG;
  constexpr int LOADS = (CHUNKS + kThreads - 1) / kThreads;  // chunks per thread per tile
  constexpr int GROUPS = TE / 16;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
  const int64_t b = blockIdx.y;
  const int64_t i0 = int64_t(blockIdx.x) * kPrefillQPB;
  const int H_I = a.H_I;
  const int64_t rowbase = b * a.T;
  const int64_t qw0 = i0 + kPrefillQPW * wid;  // this wave's first query
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- A operands: row `col` = query col/4 of the wave, head 4*hf + col%4.
  // k-slots 8g..8g+7 of k-step ks are dims 16g+8ks.. (DI = 64) or 8g.. (DI = 32).
  bf16x8_t qa[2][KSTEP];
  uint64_t qa8[2][KSTEP];  // the same slots as e4m3 codes (Q8)
  float qscale[2] = {1.0f, 1.0f};
  {
    const int64_t qi = qw0 + col / 4;
    const bf16_t* qbase = reinterpret_cast<const bf16_t*>(a.q_idx);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int h = 4 * hf + col % 4;
      const bool ok = qi < a.T && h < H_I;
      uint4 qraw[KSTEP];
      const bf16_t* qr = qbase + ((rowbase + qi) * H_I + h) * DI;
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(qr + (DI == 64 ? 16 * g + 8 * ks : 8 * g));
        qa[hf][ks] = u32x4_as_bf16x8(v);
        qraw[ks] = v;
      }
      if (Q8) {
        float part = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) part = fmaxf(part, bf16x8_absmax(qraw[ks]));
        qscale[hf] = e4m3_row_scale(part);
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) qa8[hf][ks] = bf16x8_to_e4m3x8(qraw[ks], qscale[hf]);
      }
    }
  }
  // ---- output side: the lanes of group g score query qw0 + g.
  const int64_t iq = qw0 + g;
  const bool qvalid = iq < a.T;
  int cq = 0;  // entries visible to the query
  if (qvalid) {
    const int64_t c = (a.t0 + iq + 1) / a.m;
    cq = int(c < a.N_alloc ? c : a.N_alloc);
  }
  const int need_l = cq < a.top_k ? cq : a.top_k;
  float wv[8];
#pragma unroll
  for (int h = 0; h < 8; ++h)
    wv[h] = (qvalid && h < H_I) ? (a.w ? a.w[(rowbase + iq) * H_I + h] : 1.0f) : 0.0f;
  if (Q8) {
    // The query scale of head h moves into its weight (relu(s * x) = s * relu(x)
    // for s > 0); it is held by A row 4g + h % 4, which is lane 4g + h % 4.
#pragma unroll
    for (int h = 0; h < 8; ++h) wv[h] *= __shfl(qscale[h / 4], 4 * g + h % 4);
  }
  uint64_t tau = 0ull;             // every key appended from now on is > tau
  bool active = qvalid;            // this lane's query takes part in the current pass
  // Screening score of tau: NaN admits everything, +inf (a lane whose query
  // takes no part in the current pass) all but NaN scores, which the drain drops.
  float tau_s = qvalid ? key_score(0u) : INFINITY;
  uint32_t top_hi = 0u;            // largest upper key half in the query's buffer
  int cnt = 0;                     // keys in the query's workspace buffer
  int scnt = 0;                    // pairs staged in LDS by the wave (all its queries)

  // Entries visible to the last query of this workgroup bound the sweep.
  const int64_t ilast = (i0 + kPrefillQPB < a.T ? i0 + kPrefillQPB : a.T) - 1;
  int64_t cmax64 = (a.t0 + ilast + 1) / a.m;
  if (cmax64 > a.N_alloc) cmax64 = a.N_alloc;
  const int cmax = int(cmax64);
  const int ntiles = (cmax + TE - 1) / TE;
  uint64_t* bufs = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(a.ws) + p.off_cand);
  const int cap = int(p.cap);
  uint64_t* const stg = L.stg[wid];
  const uint32_t coltag = uint32_t(col) | (uint32_t(g) << kTagShift);  // staged entry, less e0 + 16 gi

  const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(a.k_idx) + b * a.N_alloc * int64_t(DI * KB);
  // Tile prefetch registers (at most four 16-byte chunks per thread).  Every
  // thread always issues the same loads (entries past the last visible one read
  // that entry again; their scores are never candidates), so the number of loads
  // issued after any append store is fixed and the waits for those stores never
  // have to drain the prefetch too.
  static_assert(LOADS >= 1 && LOADS <= 4, "tile chunks per thread");
  uint4 pre[LOADS];
  int pid[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    pre[u] = make_uint4(0, 0, 0, 0);
    pid[u] = (tid + u * kThreads) % CHUNKS;
  }
  float psc = 1.0f;
  int ss = 1;  // entry stride of the sweep (the sample stride in the sampling pass)
  // Byte offsets of this thread's chunks (and of its scale) from the first byte
  // of a tile, fixed for a pass: a tile whose entries all lie below cmax is
  // then read from one scalar base per tile; only the last tile clamps its
  // entries one by one.  (A tile spans TE * ss < 2^31 / 128 entries, so the
  // offsets fit 32 bits.)
  uint32_t coff[LOADS], soff = 0;
  auto set_stride = [&](int stride) {
    ss = stride;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) coff[u] = uint32_t((pid[u] / CPG) * ss * (DI * KB) + (pid[u] % CPG) * 16);
    soff = uint32_t((tid & (TE - 1)) * ss) * 4u;
  };
  const float* sbytes = key_is_e4m3(KK) ? a.k_scale + b * a.N_alloc : nullptr;
  auto fetch = [&](int t) {
    if ((t * TE + TE - 1) * ss < cmax) {
      const uint8_t* tb = kbytes + int64_t(t) * (TE * ss) * (DI * KB);
#pragma unroll
      for (int u = 0; u < LOADS; ++u) pre[u] = *reinterpret_cast<const uint4*>(tb + coff[u]);
      if (key_is_e4m3(KK))
        psc = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(sbytes + int64_t(t) * (TE * ss)) + soff);
    } else {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int ge = min((t * TE + pid[u] / CPG) * ss, cmax - 1);
        pre[u] = *reinterpret_cast<const uint4*>(kbytes + int64_t(ge) * (DI * KB) + (pid[u] % CPG) * 16);
      }
      if (key_is_e4m3(KK)) psc = sbytes[min((t * TE + (tid & (TE - 1))) * ss, cmax - 1)];
    }
  };
  // Writes the prefetched chunks to LDS buffer `buf`; fp8 keys for bf16
  // products are widened to bf16 here, once per workgroup, rather than by every
  // wave that reads them.  Raw codes of 32-dim keys are placed in 8-byte slots
  // (dims 8s..8s+7 in slot s ^ ((e >> 2) & 3)), so that 16 lanes reading one
  // slot of 16 consecutive entries hit distinct banks.
  auto put = [&](int buf, int id, const uint4& v) {
    const int e = id / CPG, c = id % CPG;
    if (KK == kKeyBF16 || (Q8 && DI == 64)) {
      L.tile[buf][chunk_pos(e, c, CPE)] = v;
    } else if (Q8) {
      uint2* t8 = reinterpret_cast<uint2*>(L.tile[buf]);
      const int h = (e >> 2) & 3;
      t8[e * 4 + ((2 * c) ^ h)] = make_uint2(v.x, v.y);
      t8[e * 4 + ((2 * c + 1) ^ h)] = make_uint2(v.z, v.w);
    } else {
      uint4 lo, hi;
      e4m3x4_to_bf16x4(v.x, lo.x, lo.y);
      e4m3x4_to_bf16x4(v.y, lo.z, lo.w);
      e4m3x4_to_bf16x4(v.z, hi.x, hi.y);
      e4m3x4_to_bf16x4(v.w, hi.z, hi.w);
      L.tile[buf][chunk_pos(e, 2 * c, CPE)] = lo;
      L.tile[buf][chunk_pos(e, 2 * c + 1, CPE)] = hi;
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      if (tid + u * kThreads < CHUNKS) put(buf, pid[u], pre[u]);
    if (key_is_e4m3(KK) && tid < TE) L.scale[buf][tid] = psc;
  };
  // B operands of entry group gi (16 entries) of LDS buffer `buf`: dims
  // 16g..16g+15 (DI = 64) or 8g..8g+7 (DI = 32) of entry 16*gi + col.
  // Raw codes (Q8): dims 16g..16g+15 (DI = 64) or 8g..8g+7 (DI = 32) in b0.
  auto operands = [&](int buf, int gi, uint4& b0, uint4& b1) {
    const int e = gi * 16 + col;
    if (Q8) {
      b1 = make_uint4(0, 0, 0, 0);
      if (DI == 64) {
        b0 = L.tile[buf][chunk_pos(e, g, CPE)];
      } else {
        const uint2 v = reinterpret_cast<const uint2*>(L.tile[buf])[e * 4 + (g ^ ((e >> 2) & 3))];
        b0 = make_uint4(v.x, v.y, 0, 0);
      }
    } else if (DI == 64) {
      b0 = L.tile[buf][chunk_pos(e, 2 * g, CPE)];
      b1 = L.tile[buf][chunk_pos(e, 2 * g + 1, CPE)];
    } else {
      b0 = L.tile[buf][chunk_pos(e, g, CPE)];
      b1 = make_uint4(0, 0, 0, 0);
    }
  };
  auto products = [&](const uint4& b0, const uint4& b1, f32x4_t (&acc)[2]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
      if (Q8) {
        z = mfma16x16x32_fp8(qa8[hf][0], (uint64_t(b0.y) << 32) | b0.x, z);
        if (DI == 64) z = mfma16x16x32_fp8(qa8[hf][1], (uint64_t(b0.w) << 32) | b0.z, z);
        acc[hf] = z;
        continue;
      }
      z = mfma16x16x32(qa[hf][0], u32x4_as_bf16x8(b0), z);
      if (DI == 64) z = mfma16x16x32(qa[hf][KSTEP - 1], u32x4_as_bf16x8(b1), z);
      acc[hf] = z;
    }
  };

  // Buffer size at which a drain compacts, and the number of keys a compaction
  // keeps at least (k, or r in the sampling pass).
  int cap_pass = cap;
  int target_l = need_l;
  // Moves every pair staged by this wave into the workspace buffer of its
  // query.  A buffer that cannot take its query's staged pairs is first
  // compacted: tau rises to a bin edge that keeps between k and 5k/4 of its
  // keys, and staged pairs that do not exceed the new tau are dropped as well.
  auto drain = [&]() {
    const int ns = scnt;
    // Pairs staged per query (held by the lanes of the query's group).
    int my_ns = 0;
    for (int x0 = 0; x0 < ns; x0 += kWave) {
      const int x = x0 + lane;
      const uint32_t tag = x < ns ? uint32_t(stg[x]) >> kTagShift : 4u;
#pragma unroll
      for (int q = 0; q < kPrefillQPW; ++q) {
        const int c = __popcll(__ballot(tag == uint32_t(q)));
        if (g == q) my_ns += c;
      }
    }
#pragma unroll 1
    for (int q = 0; q < kPrefillQPW; ++q) {
      const int n = __builtin_amdgcn_readlane(cnt, 16 * q);
      const int need = __builtin_amdgcn_readlane(target_l, 16 * q);
      // A buffer of at most 5/4 of the target takes a full staging area
      // without compaction (the capacity is at least 5/4 of any target plus
      // kStage), so it is compacted only above that.
      if (n + __builtin_amdgcn_readlane(my_ns, 16 * q) > cap_pass && n > need + need / 4) {
        wait_mem();  // earlier drains of this wave have reached the buffer
        uint64_t* buf = bufs + (rowbase + qw0 + q) * cap;
        const uint64_t tq = shfl64(tau, 16 * q);
        const uint32_t tp = __builtin_amdgcn_readlane(top_hi, 16 * q);
        int kept;
        const uint64_t T = wave_threshold(buf, n, need, false, need + need / 4, tq, tp, L.hist[wid], kept);
        const int n2 = wave_compact(buf, n, T);
        if (g == q) {
          cnt = n2;
          if (T > tau) {
            tau = T;
            tau_s = key_score(uint32_t(T >> 32));
          }
        }
      }
    }
    // Rank keys are formed here, and only keys above their query's (possibly
    // raised) tau are kept.
    int nq[kPrefillQPW];
    uint32_t kmq[kPrefillQPW];
#pragma unroll
    for (int q = 0; q < kPrefillQPW; ++q) {
      nq[q] = __builtin_amdgcn_readlane(cnt, 16 * q);
      kmq[q] = 0u;
    }
    for (int x0 = 0; x0 < ns; x0 += kWave) {
      const int x = x0 + lane;
      const uint64_t sv = x < ns ? stg[x] : 0ull;
      const uint32_t tag = uint32_t(sv) >> kTagShift;
      const uint64_t tq = shfl64(tau, 16 * int(tag));
      const bool act = __shfl(int(active), 16 * int(tag)) != 0;  // NaN scores of inactive queries
      const uint64_t v = rank_key(score_key(__uint_as_float(uint32_t(sv >> 32))),
                                  uint32_t(sv) & ((1u << kTagShift) - 1u));
      const bool keep = x < ns && act && v > tq;
      int pos = 0;
#pragma unroll
      for (int q = 0; q < kPrefillQPW; ++q) {
        const bool mine = tag == uint32_t(q);
        const uint64_t bq = __ballot(keep && mine);
        if (mine) pos = nq[q] + __popcll(bq & below);
        if (keep && mine) kmq[q] = max(kmq[q], uint32_t(v >> 32));
        nq[q] += __popcll(bq);
      }
      if (keep) bufs[(rowbase + qw0 + int(tag)) * cap + pos] = v;
    }
#pragma unroll
    for (int q = 0; q < kPrefillQPW; ++q) {
      const uint32_t km = wave_max_u32(kmq[q]);
      if (g == q) {
        cnt = nq[q];
        top_hi = max(top_hi, km);
      }
    }
    scnt = 0;
    __builtin_amdgcn_wave_barrier();
  };

  // Sampling pass.  With many more visible entries than k, a first sweep over
  // every ss-th entry (about 8192 of them) finds, per query, the r-th best
  // sampled score.  The full sweep then starts with that score as its
  // threshold, which prunes about all but r * ss entries (a little over 2k)
  // from the start instead of admitting every entry until the buffer first
  // fills.  The pruning is checked afterwards: a query whose
  // full sweep kept fewer than need candidates (possible only when more than r
  // of the sampled entries rank among its true top-k) is swept again with no
  // threshold, so the result stays exact for any input.
  const bool sampling = a.top_k > 0 && cmax >= 16 * a.top_k && cmax >= 8192;
  int sstride = 2;
  while (sampling && int64_t(sstride) * 8192 < cmax) sstride *= 2;
  // r = lambda + 5 * ceil(sqrt(lambda)) + 8 sampled keys above the starting
  // threshold, lambda = ceil(need / ss) being the expected number of sampled
  // entries among the query's true top-need.  The margin trades survivors
  // against rescans: with independent scores at k = 1024 over 2^18 entries
  // (lambda = 32) a query is swept again with probability 4e-9 (about one
  // 8192-query chunk in 30000); 4 standard deviations would save another 2%
  // of the sweep but rescan one chunk in 300, and 3 one chunk in 2.
  int r_l = 0;
  {
    const int lam = (need_l + sstride - 1) / sstride;
    int sq = 0;
    while (sq * sq < lam) ++sq;
    r_l = lam + 5 * sq + 8;
  }
  bool pruned = false; // this lane's query started the full sweep above zero
#pragma unroll 1
  for (int pass = sampling ? 0 : 1; pass < 3; ++pass) {
    if (pass == 2) {
      const bool redo = qvalid && pruned && cnt < need_l;
      if (!__syncthreads_or(redo)) break;
      active = redo;
      tau_s = INFINITY;
      if (redo) {
        tau = 0ull;
        tau_s = key_score(0u);
        cnt = 0;
        top_hi = 0u;
      }
    }
    set_stride(pass == 0 ? sstride : 1);
    // The sampling pass compacts early, to about r keys, so that its threshold
    // rises fast; the full sweeps keep at least k.
    cap_pass = pass == 0 ? min(cap, max(1024, 8 * int(wave_max_u32(uint32_t(r_l))))) : cap;
    target_l = pass == 0 ? min(r_l, max(need_l, 1)) : need_l;
    const int ntp = pass == 0 ? ((cmax + ss - 1) / ss + TE - 1) / TE : ntiles;
    const int cqv = pass == 0 ? (cq + ss - 1) / ss : cq;
    // Tiles every query of the workgroup sees in full need no visibility test
    // (its first query sees the fewest entries).
    const int64_t cfirst64 = (a.t0 + i0 + 1) / a.m < a.N_alloc ? (a.t0 + i0 + 1) / a.m : a.N_alloc;
    const int cfull = pass == 0 ? (int(cfirst64) + ss - 1) / ss : int(cfirst64);
    if (ntp > 0) {
      fetch(0);
      stage(0);
      fetch(ntp > 1 ? 1 : 0);
    }
    __syncthreads();

    for (int t = 0; t < ntp; ++t) {
      const int cur = t & 1;
      const int e0 = t * TE;
      // B operands are read two groups ahead of their products: each read has
      // a group's work to land, and the reads of the 8 waves, which leave the
      // barrier together, spread over the tile instead of queueing at its start.
      constexpr int LA = 2;
      uint4 bo0[GROUPS], bo1[GROUPS];
  #pragma unroll
      for (int gi = 0; gi < LA; ++gi) operands(cur, gi, bo0[gi], bo1[gi]);
      const int lim = cqv - e0 - col;  // entry 16*gi + col of the tile is visible iff 16*gi < lim
      // The groups of the tile; FULL: every query of the workgroup sees the
      // whole tile, so the visibility test is left out.
      auto groups = [&](auto full_c) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        f32x4_t acc[2], nxt[2];
        products(bo0[0], bo1[0], acc);
  #pragma unroll
        for (int gi = 0; gi < GROUPS; ++gi) {
          if (gi + LA < GROUPS) operands(cur, gi + LA, bo0[gi + LA], bo1[gi + LA]);
          if (gi + 1 < GROUPS) products(bo0[gi + 1], bo1[gi + 1], nxt);
          const int e = gi * 16 + col;
          float s = 0.0f;
  #pragma unroll
          for (int hf = 0; hf < 2; ++hf)
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float t = fmaf(wv[4 * hf + j], relu_nan(acc[hf][j]), s);
              s = (FH || 4 * hf + j < H_I) ? t : s;
            }
          if (key_is_e4m3(KK)) s *= L.scale[cur][e];
          if (BS) s = round_bf16(s);  // screen and rank the rounded score
          // The screen admits every entry whose rank key can exceed tau (and a
          // few equal-score ones that cannot); the exact test runs when staged
          // entries are drained.  The passing lanes write their pairs to
          // consecutive staging slots in lane order.  (In full tiles the
          // compare alone is the write mask.)
          bool pass = !(s < tau_s);
          if (!FULL) pass = pass && 16 * gi < lim;
          const uint64_t m = __ballot(pass);
          if (m) {
            if (pass) {
              const uint32_t pos = __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo(uint32_t(m), uint32_t(scnt)));
              stg[pos] = (uint64_t(__float_as_uint(s)) << 32) | (uint32_t(e0 + 16 * gi) + coltag);
            }
            scnt += __popcll(m);
          }
          if (gi + 1 < GROUPS) {
            acc[0] = nxt[0];
            acc[1] = nxt[1];
          }
        }
      };
      if (e0 + TE <= cfull) groups(std::integral_constant<bool, true>());
      else groups(std::integral_constant<bool, false>());
      // The staging area is drained when it cannot take another tile.
      if (scnt > kStage - TE * kPrefillQPW) drain();
      // Tile t+1 (loaded during the previous tile) goes to the other buffer, which
      // every wave finished reading before the last barrier; each wave writes its
      // part when it is done with tile t, so the writes of the 8 waves spread out
      // instead of meeting their operand reads at the tile start.  Tile t+2 then
      // stays in flight for the whole of the next tile.
      if (t + 1 < ntp) stage(cur ^ 1);
      fetch(t + 2 < ntp ? t + 2 : ntp - 1);
      __syncthreads();
    }
    if (scnt > 0) drain();
    if (pass == 0) {
      // Starting threshold of each query: the r-th best sampled rank key with
      // its index half cleared (so every entry with that score passes).
      wait_mem();  // every drain of this wave has reached the buffers
      uint64_t t0k = 0ull;
#pragma unroll 1
      for (int q = 0; q < kPrefillQPW; ++q) {
        const int n = __builtin_amdgcn_readlane(cnt, 16 * q);
        const int need = __shfl(need_l, 16 * q);
        const int r = __shfl(r_l, 16 * q);
        const int cqq = __shfl(cq, 16 * q);
        uint64_t T = 0ull;
        if (need > 0 && cqq >= 16 * need && n >= r) {
          const uint64_t tq = shfl64(tau, 16 * q);
          const uint32_t tp = __builtin_amdgcn_readlane(top_hi, 16 * q);
          int kept;
          T = wave_threshold(bufs + (rowbase + qw0 + q) * cap, n, r, true, 0, tq, tp, L.hist[wid], kept) &
              0xffffffff00000000ull;
        }
        if (g == q) t0k = T;
      }
      tau = t0k;
      tau_s = active ? key_score(uint32_t(t0k >> 32)) : INFINITY;  // t0k = 0: NaN, admits everything
      pruned = t0k != 0ull;
      cnt = 0;
      scnt = 0;
      top_hi = 0u;
      __syncthreads();  // the tiles and staging areas are reused by the next pass
    }
  }

  // ---- final exact selection for each query of this wave
  wait_mem();  // every drain of this wave has reached the buffers
  uint32_t grp_top = top_hi;
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) grp_top = max(grp_top, __shfl_xor(grp_top, o));
#pragma unroll 1
  for (int q = 0; q < kPrefillQPW; ++q) {
    const int64_t qi = qw0 + q;
    if (qi >= a.T) break;
    const int n = __builtin_amdgcn_readlane(cnt, 16 * q);
    const int need = __shfl(need_l, 16 * q);
    const uint64_t tq = shfl64(tau, 16 * q);
    const uint32_t tp = __shfl(grp_top, 16 * q);
    const uint64_t* buf = bufs + (rowbase + qi) * cap;
    const int64_t orow = (rowbase + qi) * a.top_k;
    int kept = 0;
    uint64_t T = 1ull;  // every rank key is >= 1
    if (need > 0 && need < n) T = wave_threshold(buf, n, need, true, 0, tq, tp, L.hist[wid], kept);
    int out = 0;
    if (need > 0) {
      for (int x0 = 0; x0 < n; x0 += kWave * kBatch) {
        uint64_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int x = x0 + u * kWave + lane;
          v[u] = x < n ? buf[x] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int x = x0 + u * kWave + lane;
          const bool win = x < n && v[u] >= T;
          const uint64_t mm = __ballot(win);
          const int pos = out + __popcll(mm & below);
          if (win) {
            a.out_idx[orow + pos] = int32_t(rank_key_idx(v[u]));
            if (a.out_score) a.out_score[orow + pos] = key_score(uint32_t(v[u] >> 32));
          }
          out += __popcll(mm);
        }
      }
    }
    for (int x = out + lane; x < a.top_k; x += kWave) {
      a.out_idx[orow + x] = -1;
      if (a.out_score) a.out_score[orow + x] = -INFINITY;
    }
  }
}

template <int KK, int DI, bool FH>
void launch_prefill_bs(const IndexArgs& a, const IndexPlan& p, dim3 grid, dim3 block) {
  if (a.bf16_scores) hipLaunchKernelGGL((idx_prefill_kernel<KK, DI, FH, true>), grid, block, 0, a.stream, a, p);
  else hipLaunchKernelGGL((idx_prefill_kernel<KK, DI, FH, false>), grid, block, 0, a.stream, a, p);
}

template <int KK>
void dispatch_prefill(const IndexArgs& a, const IndexPlan& p, dim3 grid, dim3 block, bool fh) {
  if (a.d_I == 64) fh ? launch_prefill_bs<KK, 64, true>(a, p, grid, block) : launch_prefill_bs<KK, 64, false>(a, p, grid, block);
  else fh ? launch_prefill_bs<KK, 32, true>(a, p, grid, block) : launch_prefill_bs<KK, 32, false>(a, p, grid, block);
}

}  // namespace

bool prefill_path(int64_t T, int H_I, int key_kind) {
  return T >= kPrefillMinT && H_I <= 8 && key_kind != kKeyF32;
}

hipError_t launch_index_prefill(const IndexArgs& a, const IndexPlan& p) {
  const dim3 grid(unsigned((a.T + kPrefillQPB - 1) / kPrefillQPB), unsigned(a.B)), block(kThreads);
  CSA_HOST_CHECK(p.cap >= 2 * int64_t(a.top_k) + 512 && p.cap >= 4096);
  CSA_HOST_CHECK(p.off_cand >= kHeaderBytes &&
                 p.off_cand + size_t(a.B) * size_t(a.T) * size_t(p.cap) * 8 <= p.ws_bytes);
  log_dispatch("index_topk prefill: grid %u x %u of %d threads, %d queries per workgroup, buffer %lld keys",
               grid.x, grid.y, kThreads, kPrefillQPB, (long long)p.cap);
  ProfScope prof("index_topk", a.stream);
  const bool fh = a.H_I == 8;
  if (a.key_kind == kKeyBF16) dispatch_prefill<kKeyBF16>(a, p, grid, block, fh);
  else if (a.key_kind == kKeyE4M3Q8) dispatch_prefill<kKeyE4M3Q8>(a, p, grid, block, fh);
  else dispatch_prefill<kKeyE4M3>(a, p, grid, block, fh);
  return hipGetLastError();
}

}  // namespace csa
