// Lightning-Indexer scoring with streaming exact top-k for many query tokens (prefill).
//
// V4 report digest, sections 三 and 七: every query token scores all visible
// compressed entries with the indexer and keeps the top-k; in a long prefill the
// full score matrix (queries x entries) is far too large to materialise, so the
// selection is fused into the scoring sweep.
//
// Work split.  A workgroup owns 32 query tokens of one sequence (8 per wave) and
// sweeps every entry visible to any of them.  Entry keys are staged in LDS in
// tiles of 128 (16-byte chunks XOR-swizzled by entry so the MFMA operand reads
// are conflict-free) and shared by the four waves; the next tile is already in
// registers while the current one is scored.
//
// MFMA layout.  16x16x32 bf16 products with entries as columns.  A wave's query
// rows are arranged as tile pairs: tile A holds heads 0-3 and tile B heads 4-7
// of the same 4 queries (row 4*q + h), so lane (g, col) receives all 8 head dots
// of query g for entry col and forms sum_h w_h * ReLU(dot_h) without any
// cross-lane exchange.
//
// Exact top-k.  Each query keeps a candidate buffer in the workspace and a
// threshold (a 64-bit rank key: score, then lower index first).  Entries whose
// rank exceeds the threshold are appended with wave ballots, so the order is
// deterministic.  When a buffer is nearly full, one wave-local histogram pass
// raises the threshold to the lower edge of the bin holding the k-th best
// candidate and compacts the buffer; everything dropped ranks below k
// candidates already kept, so the final exact selection over the buffer gives
// the exact top-k.
#include "common.hpp"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileE = 128;  // entries per LDS tile
constexpr int kHBits = 11;   // histogram digit
constexpr int kHBins = 1 << kHBits;

struct LdsPrefill {
  uint4 tile[kTileE * 8];        // up to 128 B per entry
  float scale[kTileE];
  uint32_t hist[kWaves][kHBins];
  uint32_t cnt[kWaves][kPrefillQPW];
};

// Chunk position of chunk c of entry e (cpe chunks per entry, power of two).
__device__ __forceinline__ int chunk_pos(int e, int c, int cpe) { return e * cpe + (c ^ (e & (cpe - 1))); }

// ---------------------------------------------------------------- wave-local selection

// Radix threshold over the n keys of buf (one wave).  exact: the threshold T with
// exactly `need` keys >= T.  Otherwise T may keep more: the search stops at the
// first digit whose keys above-and-in fit in `keep_max`.  Returns T and sets kept.
__device__ uint64_t wave_threshold(const uint64_t* buf, int n, int need, bool exact, int keep_max,
                                   uint32_t* hist, int& kept) {
  const int lane = threadIdx.x & 63;
  uint64_t prefix = 0;
  int hi_bit = 64, above_total = 0;
  kept = n;
  while (hi_bit > 0) {
    const int width = hi_bit >= kHBits ? kHBits : hi_bit;
    const int shift = hi_bit - width;
    const uint32_t nb = 1u << width;
    for (int x = lane; x < kHBins; x += kWave) hist[x] = 0;
    __builtin_amdgcn_wave_barrier();
    const uint64_t hi_mask = (hi_bit >= 64) ? 0ull : (~0ull << hi_bit);
    for (int x = lane; x < n; x += kWave) {
      const uint64_t v = buf[x];
      if ((v & hi_mask) == prefix) atomicAdd(&hist[uint32_t(v >> shift) & (nb - 1u)], 1u);
    }
    __builtin_amdgcn_wave_barrier();
    // Bins in descending order, nb/64 per lane (at least one lane-bin when nb < 64).
    const uint32_t bpl = nb >= kWave ? nb / kWave : 1u;
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
    uint32_t dstar = 0, above = 0, indig = 0;
    bool mine = false;
    if (uint32_t(lane) * bpl < nb && int(ex) < need && int(inc) >= need) {
      uint32_t cum = ex;
      for (uint32_t j = 0; j < bpl; ++j) {
        const uint32_t dd = nb - 1 - (lane * bpl + j);
        const uint32_t h = hist[dd];
        if (int(cum + h) >= need) {
          dstar = dd;
          above = cum;
          indig = h;
          break;
        }
        cum += h;
      }
      mine = true;
    }
    const uint64_t who = __ballot(mine);
    const int src = __ffsll((long long)who) - 1;
    dstar = __shfl(dstar, src);
    above = __shfl(above, src);
    indig = __shfl(indig, src);
    __builtin_amdgcn_wave_barrier();
    prefix |= uint64_t(dstar) << shift;
    need -= int(above);
    above_total += int(above);
    hi_bit = shift;
    kept = above_total + int(indig);
    if (int(indig) == need) break;
    if (!exact && kept <= keep_max) break;
  }
  return prefix;
}

// Keep the keys >= T of buf[0..n) in order (in place); returns the new count.
__device__ int wave_compact(uint64_t* buf, int n, uint64_t T) {
  const int lane = threadIdx.x & 63;
  int out = 0;
  for (int x0 = 0; x0 < n; x0 += kWave) {
    const int x = x0 + lane;
    const uint64_t v = x < n ? buf[x] : 0ull;
    const bool keep = x < n && v >= T;
    const uint64_t m = __ballot(keep);
    const int pos = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    __builtin_amdgcn_wave_barrier();
    if (keep) buf[out + pos] = v;
    out += __popcll(m);
  }
  return out;
}

// ---------------------------------------------------------------- kernel

template <int KK, int DI>
__global__ __launch_bounds__(kThreads) void idx_prefill_kernel(IndexArgs a, IndexPlan p) {
  __shared__ LdsPrefill L;
  constexpr int KB = (KK == kKeyE4M3) ? 1 : 2;  // key bytes per element
  constexpr int CPE = DI * KB / 16;              // 16-byte chunks per entry
  constexpr int KSTEP = DI / 32;                 // 32-wide k-steps of one dot product
  constexpr int LOADS = kTileE * CPE / kThreads; // chunks per thread per tile
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, col = lane & 15;
  const int64_t b = blockIdx.y;
  const int64_t i0 = int64_t(blockIdx.x) * kPrefillQPB;
  const int H_I = a.H_I;
  const int64_t rowbase = b * a.T;

  // ---- per-lane query state: pair pp covers queries i0 + 8*wid + 4*pp + (0..3)
  bf16x8_t qa[2][2][KSTEP];  // [pair][head half][k-step]
  float wv[2][8];
  int64_t cq[2], iq[2];
  uint64_t tau[2] = {0ull, 0ull};
  const bf16_t* qbase = reinterpret_cast<const bf16_t*>(a.q_idx);
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    // A operand row `col`: query col/4 of the pair, head 4*hf + col%4.
    const int64_t qi = i0 + 8 * wid + 4 * pp + col / 4;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int h = 4 * hf + col % 4;
      const bool ok = qi < a.T && h < H_I;
      const bf16_t* qr = qbase + ((rowbase + qi) * H_I + h) * DI;
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *reinterpret_cast<const uint4*>(qr + (DI == 64 ? 16 * g + 8 * ks : 8 * g));
        qa[pp][hf][ks] = u32x4_as_bf16x8(v);
      }
    }
    // Output side: lane (g, col) holds query 4*pp + g of this wave.
    iq[pp] = i0 + 8 * wid + 4 * pp + g;
    const bool valid = iq[pp] < a.T;
    int64_t c = valid ? (a.t0 + iq[pp] + 1) / a.m : 0;
    cq[pp] = c < a.N_alloc ? c : a.N_alloc;
#pragma unroll
    for (int h = 0; h < 8; ++h)
      wv[pp][h] = (valid && h < H_I) ? (a.w ? a.w[(rowbase + iq[pp]) * H_I + h] : 1.0f) : 0.0f;
  }
  if (lane < kPrefillQPW) L.cnt[wid][lane] = 0;

  // Entries visible to the last query of this workgroup bound the sweep.
  const int64_t ilast = (i0 + kPrefillQPB < a.T ? i0 + kPrefillQPB : a.T) - 1;
  int64_t cmax = (a.t0 + ilast + 1) / a.m;
  if (cmax > a.N_alloc) cmax = a.N_alloc;
  const int64_t ntiles = (cmax + kTileE - 1) / kTileE;
  uint64_t* bufs = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(a.ws) + p.off_cand);
  const int cap = int(p.cap);

  const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(a.k_idx) + b * a.N_alloc * int64_t(DI * KB);
  uint4 pre[LOADS];
  float psc = 1.0f;
  auto fetch = [&](int64_t t) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int id = tid + u * kThreads, e = id / CPE, c = id % CPE;
      const int64_t ge = t * kTileE + e;
      pre[u] = ge < cmax ? *reinterpret_cast<const uint4*>(kbytes + ge * (DI * KB) + c * 16)
                         : make_uint4(0, 0, 0, 0);
    }
    if (KK == kKeyE4M3 && tid < kTileE) {
      const int64_t ge = t * kTileE + tid;
      psc = ge < cmax ? a.k_scale[b * a.N_alloc + ge] : 1.0f;
    }
  };
  if (ntiles > 0) fetch(0);

  for (int64_t t = 0; t < ntiles; ++t) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int id = tid + u * kThreads, e = id / CPE, c = id % CPE;
      L.tile[chunk_pos(e, c, CPE)] = pre[u];
    }
    if (KK == kKeyE4M3 && tid < kTileE) L.scale[tid] = psc;
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);
    const int64_t e0 = t * kTileE;
    for (int gi = 0; gi < kTileE / 16; ++gi) {
      const int e = gi * 16 + col;
      const int64_t ge = e0 + e;
      // B operands: dims 16g..16g+15 (DI = 64) or 8g..8g+7 (DI = 32) of entry e.
      uint4 b0 = make_uint4(0, 0, 0, 0), b1 = make_uint4(0, 0, 0, 0);
      if (KK == kKeyBF16) {
        if (DI == 64) {
          b0 = L.tile[chunk_pos(e, 2 * g, CPE)];
          b1 = L.tile[chunk_pos(e, 2 * g + 1, CPE)];
        } else {
          b0 = L.tile[chunk_pos(e, g, CPE)];
        }
      } else {
        if (DI == 64) {
          const uint4 raw = L.tile[chunk_pos(e, g, CPE)];
          e4m3x4_to_bf16x4(raw.x, b0.x, b0.y);
          e4m3x4_to_bf16x4(raw.y, b0.z, b0.w);
          e4m3x4_to_bf16x4(raw.z, b1.x, b1.y);
          e4m3x4_to_bf16x4(raw.w, b1.z, b1.w);
        } else {
          const uint4 raw = L.tile[chunk_pos(e, g / 2, CPE)];
          const uint32_t w0 = (g & 1) ? raw.z : raw.x, w1 = (g & 1) ? raw.w : raw.y;
          e4m3x4_to_bf16x4(w0, b0.x, b0.y);
          e4m3x4_to_bf16x4(w1, b0.z, b0.w);
        }
      }
      const float sc = (KK == kKeyE4M3) ? L.scale[e] : 1.0f;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        f32x4_t acc[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
          z = mfma16x16x32(qa[pp][hf][0], u32x4_as_bf16x8(b0), z);
          if (DI == 64) z = mfma16x16x32(qa[pp][hf][KSTEP - 1], u32x4_as_bf16x8(b1), z);
          acc[hf] = z;
        }
        float s = 0.0f;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int j = 0; j < 4; ++j) s = fmaf(wv[pp][4 * hf + j], fmaxf(acc[hf][j], 0.0f), s);
        if (KK == kKeyE4M3) s *= sc;
        const uint64_t rk = rank_key(score_key(s), uint32_t(ge));
        const bool cand = ge < cq[pp] && rk > tau[pp];
        const uint64_t m = __ballot(cand);
        if (m) {  // rare after the first tiles
          const uint32_t mg = uint32_t(m >> (16 * g)) & 0xffffu;
          const int q = 4 * pp + g;
          const int base = int(L.cnt[wid][q]);
          __builtin_amdgcn_wave_barrier();
          if (cand) {
            const int pos = __popc(mg & ((1u << col) - 1u));
            bufs[(rowbase + iq[pp]) * cap + base + pos] = rk;
          }
          if (col == 0) L.cnt[wid][q] = uint32_t(base + __popc(mg));
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
    // Raise thresholds of queries whose buffers are nearly full.
#pragma unroll 1
    for (int q = 0; q < kPrefillQPW; ++q) {
      const int n = int(L.cnt[wid][q]);
      if (n <= cap - kTileE) continue;
      const int pp = q / 4, gq = q % 4;
      const int64_t qi = i0 + 8 * wid + q;
      int64_t cqq = (a.t0 + qi + 1) / a.m;
      if (cqq > a.N_alloc) cqq = a.N_alloc;
      const int need = int(cqq < a.top_k ? cqq : a.top_k);
      uint64_t* buf = bufs + (rowbase + qi) * cap;
      wait_mem();
      int kept;
      const uint64_t T = wave_threshold(buf, n, need, false, cap / 2, L.hist[wid], kept);
      const int m2 = wave_compact(buf, n, T);
      wait_mem();
      if (lane == 0) L.cnt[wid][q] = uint32_t(m2);
      if (g == gq && T > tau[pp]) tau[pp] = T;
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  }

  // ---- final exact selection per query of this wave
#pragma unroll 1
  for (int q = 0; q < kPrefillQPW; ++q) {
    const int64_t qi = i0 + 8 * wid + q;
    if (qi >= a.T) break;
    int64_t cqq = (a.t0 + qi + 1) / a.m;
    if (cqq > a.N_alloc) cqq = a.N_alloc;
    const int need = int(cqq < a.top_k ? cqq : a.top_k);
    const int n = int(L.cnt[wid][q]);
    uint64_t* buf = bufs + (rowbase + qi) * cap;
    const int64_t orow = (rowbase + qi) * a.top_k;
    wait_mem();
    int kept = 0;
    uint64_t T = 1ull;
    if (need > 0 && need < n) T = wave_threshold(buf, n, need, true, 0, L.hist[wid], kept);
    int out = 0;
    if (need > 0) {
      for (int x0 = 0; x0 < n; x0 += kWave) {
        const int x = x0 + lane;
        const uint64_t v = x < n ? buf[x] : 0ull;
        const bool win = x < n && v >= T;
        const uint64_t mm = __ballot(win);
        const int pos = __popcll(mm & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        if (win) {
          a.out_idx[orow + out + pos] = int32_t(rank_key_idx(v));
          if (a.out_score) a.out_score[orow + out + pos] = key_score(uint32_t(v >> 32));
        }
        out += __popcll(mm);
      }
    }
    for (int x = out + lane; x < a.top_k; x += kWave) {
      a.out_idx[orow + x] = -1;
      if (a.out_score) a.out_score[orow + x] = -INFINITY;
    }
  }
}

}  // namespace

bool prefill_path(int64_t T, int H_I, int key_kind) {
  return T >= kPrefillMinT && H_I <= 8 && key_kind != kKeyF32;
}

hipError_t launch_index_prefill(const IndexArgs& a, const IndexPlan& p) {
  const dim3 grid(unsigned((a.T + kPrefillQPB - 1) / kPrefillQPB), unsigned(a.B)), block(kThreads);
  ProfScope prof("index_topk", a.stream);
  if (a.key_kind == kKeyBF16) {
    if (a.d_I == 64) hipLaunchKernelGGL((idx_prefill_kernel<kKeyBF16, 64>), grid, block, 0, a.stream, a, p);
    else hipLaunchKernelGGL((idx_prefill_kernel<kKeyBF16, 32>), grid, block, 0, a.stream, a, p);
  } else {
    if (a.d_I == 64) hipLaunchKernelGGL((idx_prefill_kernel<kKeyE4M3, 64>), grid, block, 0, a.stream, a, p);
    else hipLaunchKernelGGL((idx_prefill_kernel<kKeyE4M3, 32>), grid, block, 0, a.stream, a, p);
  }
  return hipGetLastError();
}

}  // namespace csa
