// DeepSelect row-wise top-k: HIP kernels for gfx950 (CDNA4, 64-lane waves).
//
// Method (DeepSelect design note, "Algorithm"): a threshold T, blocks of B elements read
// once in a random order independent of the data, a filter that appends every element
// beating T to an on-chip candidate buffer, a radix-select compaction back to k entries
// whenever the buffer reaches k + B2 (which also raises T to the smallest survivor), and a
// final compaction. The split-row path (design note, "Implementation", cluster paragraph)
// runs the same method on slices of a row and merges the slices' survivors with it again.
//
// Order used everywhere: an element is the pair (value, index); larger value first,
// +0 before -0, then smaller index first. On the device an element's value is replaced
// by an order-preserving unsigned "key" (tutorial chapter section 4.6: positive values get
// their sign bit flipped, negative values all bits inverted), and a pair by the 64-bit
// composite (key << 32) | ~index, so every comparison is an integer comparison.
//
// MI355X mapping:
//  * one workgroup (2-8 waves) per (row, slice); every lane streams 16-byte raw buffer
//    loads, one wave covers 1 KiB per chunk, and each wave keeps a ring of chunks in
//    flight that runs ahead across block boundaries and across compactions;
//  * the filter compares raw bit patterns against a per-block integer threshold (no
//    key transform and no float compare on the streaming path); the per-element hit
//    masks become 64-lane SGPR masks, positions come from mbcnt, and one LDS atomic per
//    wave per block reserves buffer space;
//  * barriers are LDS-only (s_barrier with workgroup/local fences), so in-flight global
//    loads are never drained by a barrier;
//  * the compaction is an LDS radix select over the composite with 8-bit digits placed
//    below the common prefix of the buffer (found by a wave OR/AND reduction), a
//    triple-buffered histogram, and a per-wave redundant bin scan, so one barrier is
//    needed per digit; survivors ping-pong between two k-entry segments.
#include "ds_internal.h"

namespace ds {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for raw (untyped) dword buffers on the gfx9 family.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kSentinelIdx = 0xFFFFFFFFu;  // with key 0: ranks below every real element

__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), base));
}

__device__ __forceinline__ uint32_t popc(uint64_t m) { return static_cast<uint32_t>(__popcll(m)); }

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Value held by lane (lane ^ m), m a power of two below 64. Lane mappings (checked on
// gfx950): quad_perm 0xB1 / 0x4E swap neighbours at distance 1 / 2, row_ror:8 swaps the
// halves of a 16-lane row, ds_swizzle in bit-mask mode xors the lane id within 32 lanes,
// and the permlane16/32 swaps exchange 16-lane rows / 32-lane halves.
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, uint32_t m, uint32_t lane) {
  switch (m) {
    case 1: return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);
    case 4: return __builtin_amdgcn_ds_swizzle(v, 0x1F | (4 << 10));
    case 8: return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, false);
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16u) ? p[0] : p[1];
    }
    default: {
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32u) ? p[0] : p[1];
    }
  }
}

__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, uint32_t m, uint32_t lane) {
  const uint32_t lo = xor_lane(static_cast<uint32_t>(v), m, lane);
  const uint32_t hi = xor_lane(static_cast<uint32_t>(v >> 32), m, lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max64(uint64_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t m = 1; m < 64; m <<= 1) {
    const uint64_t o = xor_lane64(v, m, lane);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_min64(uint64_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t m = 1; m < 64; m <<= 1) {
    const uint64_t o = xor_lane64(v, m, lane);
    v = o < v ? o : v;
  }
  return v;
}

// Inclusive prefix sum over the 64 lanes (row shifts within 16-lane rows, then the row
// broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);
  return x;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, uint32_t l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), l);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// --------------------------------------------------------------------------- keys
// Order-preserving key of a raw element (bf16: the 16 bits in the low half).
template <int DT>
__device__ __forceinline__ uint32_t key_of_raw(uint32_t raw) {
  if constexpr (DT == DS_BF16) {
    const uint32_t neg = static_cast<uint32_t>(static_cast<int32_t>(raw << 16) >> 31);
    return raw ^ ((neg & 0x7FFFu) | 0x8000u);
  } else {
    const uint32_t neg = static_cast<uint32_t>(static_cast<int32_t>(raw) >> 31);
    return raw ^ ((neg & 0x7FFFFFFFu) | 0x80000000u);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t raw_of_key(uint32_t key) {
  if constexpr (DT == DS_BF16) {
    return key ^ ((key & 0x8000u) ? 0x8000u : 0xFFFFu);
  } else {
    return key ^ ((key & 0x80000000u) ? 0x80000000u : 0xFFFFFFFFu);
  }
}

// --------------------------------------------------------------------------- block order
// Keyed Feistel bijection on [0, 2^b) (b the smallest even width >= 2 with 2^b >= m),
// four rounds with the lowbias32 integer hash as round function, restricted to [0, m)
// by cycle walking. Round keys come from (seed, row, slice) through the splitmix64
// finaliser. The walk ends because the permutation's cycle through i returns to i < m.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

struct BlockOrder {
  uint32_t key[4];
  uint32_t half, mask, m;

  __device__ void init(uint64_t seed, uint32_t row, uint32_t slice, uint32_t m_) {
    constexpr uint64_t G = 0x9E3779B97F4A7C15ull;
    uint64_t h = mix64(seed + G * (static_cast<uint64_t>(row) + 1));
    h = mix64(h + G * (static_cast<uint64_t>(slice) + 1));
#pragma unroll
    for (int r = 0; r < 4; ++r) key[r] = static_cast<uint32_t>(mix64(h + G * static_cast<uint64_t>(r + 1)));
    uint32_t b = 2;
    while ((1u << b) < m_) b += 2;
    half = b / 2;
    mask = (1u << half) - 1;
    m = m_;
  }

  __device__ __forceinline__ uint32_t at(uint32_t i) const {
    if (m <= 1) return 0;
    uint32_t y = i;
    do {
      uint32_t l = y >> half, r = y & mask;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t t = l ^ (lowbias32(r ^ key[q]) & mask);
        l = r;
        r = t;
      }
      y = (l << half) | r;
    } while (y >= m);
    return y;
  }
};

// --------------------------------------------------------------------------- shared state
constexpr int kMaxWaves = 16;
constexpr uint32_t kBins = 512;      // histogram bins of one radix pass
constexpr uint32_t kListCap = 64;    // pivot-bin entries resolved by one wave

struct Scalars {
  uint32_t app_count;               // entries appended since the last compaction
  uint32_t outpos;                  // scatter cursor of the running compaction
  uint32_t listpos;                 // pivot-list cursor of the running compaction
  uint32_t pad0;
  uint32_t slot[2][kMaxWaves];      // per-wave end of its reservation, by block parity
  uint64_t red[kMaxWaves][2];       // per-wave min / max composites
  uint2 list[kListCap];             // entries of the pivot bin
  unsigned long long reads;         // counters (stats runs only)
  unsigned long long index_sum;
};

struct Thr {
  uint32_t key, idx;
};

__device__ __forceinline__ uint64_t comp_of(uint2 e) {
  return (static_cast<uint64_t>(e.x) << 32) | static_cast<uint32_t>(~e.y);
}

__device__ __forceinline__ uint2 entry_of(uint64_t c) {
  return make_uint2(static_cast<uint32_t>(c >> 32), ~static_cast<uint32_t>(c));
}

__device__ __forceinline__ uint32_t bitlen64(uint64_t v) { return v ? 64u - static_cast<uint32_t>(__builtin_clzll(v)) : 0u; }

// Every wave scans the same kBins-bin histogram from the top bin down and finds the bin that
// holds the `need`-th best entry: `above` entries lie in higher bins, `cnt` in that bin.
__device__ __forceinline__ void scan_select(const uint32_t* h, uint32_t need, uint32_t lane, uint32_t& bin,
                                            uint32_t& above, uint32_t& cnt) {
  constexpr uint32_t PER = kBins / 64;  // 8 bins per lane, lane 0 holds the highest
  const uint32_t top = kBins - 1u - PER * lane;
  const uint4 qa = *reinterpret_cast<const uint4*>(h + top - 7);
  const uint4 qb = *reinterpret_cast<const uint4*>(h + top - 3);
  const uint32_t c[PER] = {qb.w, qb.z, qb.y, qb.x, qa.w, qa.z, qa.y, qa.x};  // bins top, top-1, ...
  uint32_t s = 0;
#pragma unroll
  for (uint32_t i = 0; i < PER; ++i) s += c[i];
  const uint32_t incl = wave_incl_scan(s);
  const uint64_t ge = ballot(incl >= need);
  const uint32_t src = ge ? static_cast<uint32_t>(__builtin_ctzll(ge)) : 63u;
  uint32_t acc = incl - s, b = top - (PER - 1), a = acc, n = c[PER - 1];
  bool found = false;
#pragma unroll
  for (uint32_t i = 0; i < PER; ++i) {
    if (!found && acc + c[i] >= need) {
      found = true;
      b = top - i;
      a = acc;
      n = c[i];
    }
    acc += c[i];
  }
  bin = __builtin_amdgcn_readlane(b, src);
  above = __builtin_amdgcn_readlane(a, src);
  cnt = __builtin_amdgcn_readlane(n, src);
}

// Radix-select compaction.
//
// Reduces the nsurv survivors in `sin` plus the napp appended entries in `app` to the k best
// under the composite order and writes them (unordered) to `sout`. Returns the smallest kept
// composite (the new threshold) in `thr` and the largest in `maxc`.
//
// The search runs on the 64-bit composite c = (key << 32) | ~index over a window
// [lo, hi] that holds every entry: a kBins-bin histogram of (c - lo) >> shift (entries
// above hi fall in the top bin) locates the bin of the k-th best; while that bin holds more
// than kListCap entries the window shrinks to it and the histogram repeats; then the
// entries above the bin are scattered to `sout`, the bin's entries are gathered in a short
// list, and every wave ranks that list to pick the rest and the threshold.
// First call (nsurv == 0): one extra pass turns the raw entries into keys and measures the
// window. Later calls: the window is [previous threshold, previous maximum] and the raw ->
// key step is folded into the first histogram pass.
// RAW: appended entries hold raw element bits (bf16: in the high half).
template <int DT, int WAVES, bool RAW>
__device__ void compact(const uint2* sin, uint32_t nsurv, uint2* app, uint32_t napp, uint2* sout, uint32_t k,
                        Scalars& sc, uint32_t* hist3, uint32_t& hctr, uint64_t& thr, uint64_t& maxc) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t n = nsurv + napp;

  if (n <= k) {  // keep everything (only the final call can get here)
    for (uint32_t i = tid; i < k; i += NT) {
      uint2 e = make_uint2(0, kSentinelIdx);
      if (i < nsurv) {
        e = sin[i];
      } else if (i < n) {
        e = app[i - nsurv];
        if constexpr (RAW) e.x = key_of_raw<DT>(DT == DS_BF16 ? (e.x >> 16) : e.x);
      }
      sout[i] = e;
    }
    lds_sync();
    return;
  }

  uint64_t lo, hi;
  bool raw_pending = RAW;
  if (nsurv == 0) {
    uint64_t mn = ~0ull, mx = 0;
    for (uint32_t i = tid; i < n; i += NT) {
      uint2 e = app[i];
      if constexpr (RAW) {
        e.x = key_of_raw<DT>(DT == DS_BF16 ? (e.x >> 16) : e.x);
        app[i].x = e.x;
      }
      const uint64_t c = comp_of(e);
      mn = c < mn ? c : mn;
      mx = c > mx ? c : mx;
    }
    mn = wave_min64(mn, lane);
    mx = wave_max64(mx, lane);
    if (lane == 0) {
      sc.red[wave][0] = mn;
      sc.red[wave][1] = mx;
    }
    if (tid == 0) {
      sc.app_count = 0;
      sc.outpos = 0;
      sc.listpos = 0;
    }
    lds_sync();
    lo = ~0ull;
    hi = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      lo = sc.red[w][0] < lo ? sc.red[w][0] : lo;
      hi = sc.red[w][1] > hi ? sc.red[w][1] : hi;
    }
    raw_pending = false;
  } else {
    lo = thr;
    hi = maxc;
    if (tid == 0) {  // every wave passed the block barrier after its appends
      sc.app_count = 0;
      sc.outpos = 0;
      sc.listpos = 0;
    }
  }

  // histogram passes, shrinking [lo, hi] to the bin of the k-th best
  uint32_t need = k, above_total = 0, cnt = 0;
  uint64_t plo = lo, phi = hi;  // current pivot window
  bool top_open = nsurv != 0;   // entries above hi may exist (they fall in the top bin)
  uint64_t seen_max = 0;
  for (;;) {
    const uint32_t shift = bitlen64(phi - plo) > 9 ? bitlen64(phi - plo) - 9 : 0;
    uint32_t* h = hist3 + kBins * (hctr % 3u);
    uint32_t* hn = hist3 + kBins * ((hctr + 1u) % 3u);
    for (uint32_t b = tid; b < kBins; b += NT) hn[b] = 0;
    uint64_t mx = 0;
    for (uint32_t i = tid; i < n; i += NT) {
      uint2 e;
      if (i < nsurv) {
        e = sin[i];
      } else {
        e = app[i - nsurv];
        if (raw_pending) {
          e.x = key_of_raw<DT>(DT == DS_BF16 ? (e.x >> 16) : e.x);
          app[i - nsurv].x = e.x;
        }
      }
      const uint64_t c = comp_of(e);
      mx = c > mx ? c : mx;
      if (c >= plo && (c <= phi || top_open)) {
        const uint64_t d = (c > phi ? phi : c) - plo;
        atomicAdd(&h[static_cast<uint32_t>(d >> shift)], 1u);
      }
    }
    raw_pending = false;
    mx = wave_max64(mx, lane);
    if (lane == 0) sc.red[wave][1] = mx;
    lds_sync();
    ++hctr;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) seen_max = sc.red[w][1] > seen_max ? sc.red[w][1] : seen_max;
    uint32_t bin, above;
    scan_select(h, need, lane, bin, above, cnt);
    need -= above;
    above_total += above;
    const uint64_t nlo = plo + (static_cast<uint64_t>(bin) << shift);
    const bool open_bin = top_open && (bin == kBins - 1u || ((phi - plo) >> shift) == bin);
    uint64_t nhi = plo + ((static_cast<uint64_t>(bin) + 1u) << shift) - 1u;
    if (nhi > phi || nhi < nlo) nhi = phi;
    plo = nlo;
    phi = open_bin ? seen_max : nhi;
    top_open = false;
    // A chosen open bin widens the window to the true maximum, so it is refined again even
    // when this pass had single-composite bins.
    if (cnt <= kListCap || (shift == 0 && !open_bin)) break;
  }

  // scatter: everything above the pivot window is kept; the window's entries go to the list
  // (cnt > kListCap only if composites repeat, which real entries never do; the list then
  // keeps its first kListCap entries and the call still ends)
  cnt = cnt < kListCap ? cnt : kListCap;
  const uint32_t iters = (n + NT - 1) / NT;
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t i = it * NT + tid;
    uint2 e = make_uint2(0, kSentinelIdx);
    uint64_t c = 0;
    if (i < n) {
      e = i < nsurv ? sin[i] : app[i - nsurv];
      c = comp_of(e);
    }
    const bool up = i < n && c > phi;
    const bool mid = i < n && c >= plo && c <= phi;
    const uint64_t bu = ballot(up), bm = ballot(mid);
    if (bu | bm) {
      uint32_t b0 = 0, b1 = 0;
      if (lane == 0) {
        if (bu) b0 = atomicAdd(&sc.outpos, popc(bu));
        if (bm) b1 = atomicAdd(&sc.listpos, popc(bm));
      }
      b0 = uni(b0);
      b1 = uni(b1);
      if (up) {
        const uint32_t q = mbcnt(bu, b0);
        if (q < k) sout[q] = e;
      }
      if (mid) {
        const uint32_t q = mbcnt(bm, b1);
        if (q < kListCap) sc.list[q] = e;
      }
    }
  }
  lds_sync();

  // every wave ranks the short list: the `need` best of its cnt entries are kept
  const uint64_t mine = lane < cnt ? comp_of(sc.list[lane]) : 0ull;
  uint32_t rank = 0;
  for (uint32_t m = 0; m < cnt; ++m) rank += readlane64(mine, m) > mine ? 1u : 0u;
  const bool keep = lane < cnt && rank < need;
  if (wave == 0 && keep) sout[above_total + rank] = entry_of(mine);
  const uint64_t piv = ballot(lane < cnt && rank == need - 1u);
  thr = readlane64(mine, piv ? static_cast<uint32_t>(__builtin_ctzll(piv)) : 0u);
  maxc = seen_max;
}

// One compare-exchange stage (SIZE, STRIDE) of a bitonic sort of NT*E 64-bit keys, best first,
// held E per thread in registers (element t*E + j in thread t). Partners closer than E are in
// the same thread, closer than 64*E in the same wave (lane exchanges); farther partners go
// through `xbuf` (NT*E slots of LDS) between two barriers. Recurses through all later stages.
template <int WAVES, int E, uint32_t SIZE, uint32_t STRIDE>
__device__ __forceinline__ void bitonic_stages(uint64_t (&v)[E], uint64_t* xbuf, uint32_t tid, uint32_t lane) {
  constexpr uint32_t TOTAL = WAVES * 64 * E;
  if constexpr (STRIDE < static_cast<uint32_t>(E)) {
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      if ((j & STRIDE) == 0) {
        const bool desc = ((tid * E + j) & SIZE) == 0;
        const uint64_t a = v[j], b = v[j | STRIDE];
        const bool sw = desc ? b > a : a > b;
        v[j] = sw ? b : a;
        v[j | STRIDE] = sw ? a : b;
      }
    }
  } else if constexpr (STRIDE < 64u * E) {
    constexpr uint32_t M = STRIDE / E;
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      const uint32_t e = tid * E + j;
      const bool take_max = ((e & STRIDE) == 0) == ((e & SIZE) == 0);
      const uint64_t o = xor_lane64(v[j], M, lane);
      v[j] = take_max ? (o > v[j] ? o : v[j]) : (o < v[j] ? o : v[j]);
    }
  } else {
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) xbuf[tid * E + j] = v[j];
    lds_sync();
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      const uint32_t e = tid * E + j;
      const bool take_max = ((e & STRIDE) == 0) == ((e & SIZE) == 0);
      const uint64_t o = xbuf[e ^ STRIDE];
      v[j] = take_max ? (o > v[j] ? o : v[j]) : (o < v[j] ? o : v[j]);
    }
    lds_sync();
  }
  if constexpr (STRIDE > 1)
    bitonic_stages<WAVES, E, SIZE, STRIDE / 2>(v, xbuf, tid, lane);
  else if constexpr (SIZE < TOTAL)
    bitonic_stages<WAVES, E, SIZE * 2, SIZE>(v, xbuf, tid, lane);
}

// Sort the k entries of `fin` (padded with sentinels to NT*E) best first and store the first k.
template <int DT, int WAVES, int E>
__device__ void sort_store_e(const uint2* fin, uint64_t* xbuf, uint32_t k, void* out_vals, int32_t* out_idx,
                             uint64_t row) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  uint64_t v[E];
#pragma unroll
  for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
    const uint32_t e = tid * E + j;
    v[j] = e < k ? comp_of(fin[e]) : 0ull;
  }
  bitonic_stages<WAVES, E, 2, 1>(v, xbuf, tid, lane);
#pragma unroll
  for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
    const uint32_t e = tid * E + j;
    if (e < k) {
      const uint2 en = entry_of(v[j]);
      if (out_vals) {
        if constexpr (DT == DS_BF16)
          static_cast<uint16_t*>(out_vals)[row * k + e] = static_cast<uint16_t>(raw_of_key<DT>(en.x));
        else
          static_cast<uint32_t*>(out_vals)[row * k + e] = raw_of_key<DT>(en.x);
      }
      if (out_idx) out_idx[row * k + e] = static_cast<int32_t>(en.y);
    }
  }
}

// Bitonic sort in LDS (one barrier per stage), for k above four entries per thread: sorts cap
// (a power of two >= k) composites in `xbuf`, best first, and stores the first k.
template <int DT, int WAVES>
__device__ void sort_store_lds(const uint2* fin, uint64_t* xbuf, uint32_t k, void* out_vals, int32_t* out_idx,
                               uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x;
  uint32_t cap = 1;
  while (cap < k) cap <<= 1;
  for (uint32_t i = tid; i < cap; i += NT) xbuf[i] = i < k ? comp_of(fin[i]) : 0ull;
  lds_sync();
  for (uint32_t size = 2; size <= cap; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t q = tid; q < cap / 2; q += NT) {
        const uint32_t i = ((q & ~(stride - 1)) << 1) | (q & (stride - 1));
        const uint32_t j = i + stride;
        const uint64_t a = xbuf[i], b = xbuf[j];
        const bool desc = (i & size) == 0;
        if (desc ? b > a : a > b) {
          xbuf[i] = b;
          xbuf[j] = a;
        }
      }
      lds_sync();
    }
  }
  for (uint32_t i = tid; i < k; i += NT) {
    const uint2 en = entry_of(xbuf[i]);
    if (out_vals) {
      if constexpr (DT == DS_BF16)
        static_cast<uint16_t*>(out_vals)[row * k + i] = static_cast<uint16_t>(raw_of_key<DT>(en.x));
      else
        static_cast<uint32_t*>(out_vals)[row * k + i] = raw_of_key<DT>(en.x);
    }
    if (out_idx) out_idx[row * k + i] = static_cast<int32_t>(en.y);
  }
}

// `xbuf` needs max(NT, pow2 >= k) 64-bit slots; `fin` must be visible to every thread.
template <int DT, int WAVES>
__device__ void sort_and_store(uint64_t* xbuf, const uint2* fin, uint32_t k, void* out_vals, int32_t* out_idx,
                               uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  if (k <= NT)
    sort_store_e<DT, WAVES, 1>(fin, xbuf, k, out_vals, out_idx, row);
  else if (k <= 2 * NT)
    sort_store_e<DT, WAVES, 2>(fin, xbuf, k, out_vals, out_idx, row);
  else if (k <= 4 * NT)
    sort_store_e<DT, WAVES, 4>(fin, xbuf, k, out_vals, out_idx, row);
  else
    sort_store_lds<DT, WAVES>(fin, xbuf, k, out_vals, out_idx, row);
}

// Integer compare values for the streaming filter, from the threshold pair (key, idx).
// mode 1: hit <=> (int)score > thr; mode 2: hit <=> score < thr; "strict" is used for
// blocks after the threshold's index, "non-strict" (ties win) for blocks before it.
// bf16 scores carry the element in the high 16 bits.
template <int DT>
__device__ __forceinline__ void filter_thresholds(Thr t, uint32_t& mode, uint32_t& thr_s, uint32_t& thr_n) {
  const uint32_t raw = raw_of_key<DT>(t.key);
  if constexpr (DT == DS_BF16) {
    if ((raw & 0x8000u) == 0) {
      mode = 1;
      thr_s = ((raw + 1u) << 16) - 1u;
      thr_n = (raw << 16) - 1u;
    } else {
      mode = 2;
      thr_s = raw << 16;
      thr_n = (raw + 1u) << 16;
    }
  } else {
    if ((raw & 0x80000000u) == 0) {
      mode = 1;
      thr_s = raw;
      thr_n = raw - 1u;
    } else {
      mode = 2;
      thr_s = raw;
      thr_n = raw + 1u;
    }
  }
}

// --------------------------------------------------------------------------- select kernel
template <int DT, int WAVES, int CPW, int PD>
__global__ __launch_bounds__(WAVES * 64) void select_kernel(SelectParams p) {
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t EB = DT == DS_BF16 ? 2 : 4;
  constexpr uint32_t VEC = 16 / EB;
  constexpr uint32_t CHUNK = 64 * VEC;
  constexpr uint32_t B = WAVES * CPW * CHUNK;

  extern __shared__ __attribute__((aligned(16))) uint2 lds[];
  __shared__ Scalars sc;

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t row = blockIdx.x / static_cast<uint32_t>(p.slices);
  const uint32_t slice = blockIdx.x % static_cast<uint32_t>(p.slices);
  const uint32_t slice_lo = slice * static_cast<uint32_t>(p.slice_len);
  const uint32_t len = static_cast<uint32_t>(min(p.slice_len, p.n - static_cast<int64_t>(slice_lo)));
  const uint32_t m = (len + B - 1) / B;
  const uint32_t k = static_cast<uint32_t>(p.k);
  const uint32_t B2 = static_cast<uint32_t>(p.slack);
  const bool stats = p.stats != nullptr;

  uint2* const surv0 = lds;
  uint2* const surv1 = lds + k;
  uint2* const app_warm = lds + k;
  uint2* const app_main = lds + 2 * k;
  uint32_t* const hist3 = reinterpret_cast<uint32_t*>(lds + ((2 * k + B2 + B + 1u) & ~1u));  // 16-byte aligned

  for (uint32_t i = tid; i < 3u * kBins; i += NT) hist3[i] = 0;
  if (tid == 0) {
    sc.app_count = 0;
    sc.outpos = 0;
    sc.reads = 0;
    sc.index_sum = 0;
  }

  const uint8_t* base = p.x + static_cast<uint64_t>(row) * p.row_stride_bytes + static_cast<uint64_t>(slice_lo) * EB;
  // Range = the slice rounded up to whole 16-byte chunks: the hardware checks whole dwords, so
  // an exact byte count would zero the dword that holds a bf16 row's odd last element. Row
  // starts are 16-byte aligned, so the rounded range never leaves the row's last chunk.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(base), 0, static_cast<int>((len * EB + 15u) & ~15u), kRsrcWord3);
  BlockOrder ord;
  ord.init(p.seed, row, slice, m);

  // threshold state (uniform across the workgroup)
  uint32_t mode = 0, thr_s = 0, thr_n = 0, t_idx = 0;
  uint64_t thr_c = 0, maxc = 0;
  uint32_t nsurv = 0, cur = 0, napp = 0, hctr = 0;
  // counters (thread-uniform; used when stats are requested)
  uint64_t st_a = 0, st_r = 0, st_w = 0, st_max = 0, st_mono = 1, my_reads = 0, my_jsum = 0;

  u32x4 ring[PD][CPW];
  uint32_t bids[PD];
#pragma unroll
  for (uint32_t d = 0; d < PD; ++d) {
    if (d < m) {
      const uint32_t b = ord.at(d);
      bids[d] = b;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t)
        ring[d][t] = load16(rs, (b * B + (wave + t * WAVES) * CHUNK + lane * VEC) * EB);
    }
  }
  lds_sync();

  for (uint32_t i0 = 0; i0 < m; i0 += PD) {
#pragma unroll
    for (uint32_t d = 0; d < PD; ++d) {
      const uint32_t i = i0 + d;
      if (i >= m) break;
      const uint32_t bid = bids[d];
      u32x4 v[CPW];
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) v[t] = ring[d][t];
      if (i + PD < m) {
        const uint32_t nb = ord.at(i + PD);
        bids[d] = nb;
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t)
          ring[d][t] = load16(rs, (nb * B + (wave + t * WAVES) * CHUNK + lane * VEC) * EB);
      }

      // ---- filter: hit masks for every element slot of every chunk of this wave
      const uint32_t blk_lo = bid * B;
      const bool strict = slice_lo + blk_lo > t_idx;
      const uint32_t thr = strict ? thr_s : thr_n;
      uint32_t s[CPW][VEC];
      bool h[CPW][VEC];
      uint64_t mk[CPW][VEC];
      uint32_t tot = 0;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) {
        const uint32_t off = blk_lo + (wave + t * WAVES) * CHUNK;
        if constexpr (DT == DS_BF16) {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) {
            s[t][2 * q] = v[t][q] << 16;
            s[t][2 * q + 1] = v[t][q];
          }
        } else {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) s[t][q] = v[t][q];
        }
#pragma unroll
        for (uint32_t e = 0; e < VEC; ++e) {
          h[t][e] = mode == 0 ? true
                    : mode == 1 ? static_cast<int32_t>(s[t][e]) > static_cast<int32_t>(thr)
                                : s[t][e] < thr;
        }
        uint32_t nval = VEC;
        if (off + CHUNK > len) {  // the slice's tail chunk: only [0, len) is valid
          const uint32_t first = off + lane * VEC;
          nval = first >= len ? 0u : min(VEC, len - first);
#pragma unroll
          for (uint32_t e = 0; e < VEC; ++e) h[t][e] = h[t][e] && e < nval;
        }
        if (stats) {
          const uint64_t j0 = slice_lo + off + lane * VEC;
          my_reads += nval;
          my_jsum += nval * j0 + (static_cast<uint64_t>(nval) * (nval - 1)) / 2;
        }
#pragma unroll
        for (uint32_t e = 0; e < VEC; ++e) {
          mk[t][e] = ballot(h[t][e]);
          tot += popc(mk[t][e]);
        }
      }

      // ---- append: one reservation per wave per block
      uint32_t pos = 0;
      if (lane == 0) pos = atomicAdd(&sc.app_count, tot);
      pos = uni(pos);
      if (lane == 0) sc.slot[i & 1u][wave] = pos + tot;
      if (tot) {
        uint2* const app = nsurv ? app_main : app_warm;
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) {
          const uint32_t jl = slice_lo + blk_lo + (wave + t * WAVES) * CHUNK + lane * VEC;
#pragma unroll
          for (uint32_t e = 0; e < VEC; ++e) {
            if (mk[t][e]) {
              const uint32_t q = mbcnt(mk[t][e], pos);
              if (h[t][e]) app[q] = make_uint2(s[t][e], jl + e);
              pos += popc(mk[t][e]);
            }
          }
        }
      }
      lds_sync();

      // ---- compaction test after the whole block
      uint32_t cnt = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) cnt = max(cnt, sc.slot[i & 1u][w]);
      napp = cnt;
      st_max = max(st_max, static_cast<uint64_t>(nsurv + napp));
      if (nsurv + napp >= k + B2) {
        uint2* const sout = nsurv ? (cur ? surv0 : surv1) : surv0;
        const uint2* const sin = cur ? surv1 : surv0;
        const uint64_t prev_c = thr_c;
        compact<DT, WAVES, true>(sin, nsurv, nsurv ? app_main : app_warm, napp, sout, k, sc, hist3, hctr, thr_c,
                                 maxc);
        st_a += napp;
        st_w += nsurv + napp;
        st_r += 1;
        if (thr_c < prev_c) st_mono = 0;
        cur = nsurv ? (cur ^ 1u) : 0u;
        nsurv = k;
        napp = 0;
        t_idx = ~static_cast<uint32_t>(thr_c);
        filter_thresholds<DT>(Thr{static_cast<uint32_t>(thr_c >> 32), t_idx}, mode, thr_s, thr_n);
      }
    }
  }

  // ---- final compaction
  uint2* const fin = nsurv ? (cur ? surv0 : surv1) : surv0;
  {
    const uint2* const sin = cur ? surv1 : surv0;
    compact<DT, WAVES, true>(sin, nsurv, nsurv ? app_main : app_warm, napp, fin, k, sc, hist3, hctr, thr_c, maxc);
    st_a += napp;
    st_w += nsurv + napp;
  }
  lds_sync();

  if (stats) {
    for (uint32_t o = 32; o > 0; o >>= 1) {
      my_reads += __shfl_xor(my_reads, o);
      my_jsum += __shfl_xor(my_jsum, o);
    }
    if (lane == 0) {
      atomicAdd(&sc.reads, static_cast<unsigned long long>(my_reads));
      atomicAdd(&sc.index_sum, static_cast<unsigned long long>(my_jsum));
    }
    lds_sync();
    if (tid == 0) {
      ds_stats* o = p.stats + blockIdx.x;
      o->appended = st_a;
      o->compactions = st_r;
      o->work = st_w;
      o->max_len = st_max;
      o->reads = sc.reads;
      o->index_sum = sc.index_sum;
      o->monotone = st_mono;
      o->slice_lo = slice_lo;
      o->slice_len = len;
      o->block = B;
      o->slack = B2;
      o->reserved = 0;
    }
  }

  if (p.slices == 1) {
    sort_and_store<DT, WAVES>(reinterpret_cast<uint64_t*>(app_main), fin, k, p.out_vals, p.out_idx, row);
  } else {
    uint2* const dst = p.ws + static_cast<uint64_t>(row) * p.ws_row_entries + static_cast<uint64_t>(slice) * k;
    for (uint32_t i = tid; i < k; i += NT) dst[i] = fin[i];
  }
}

// --------------------------------------------------------------------------- merge kernel
// DeepSelect again, over the slices' survivors of one row: entries are already (key, index)
// pairs; a 16-byte lane load carries two of them.
template <int DT, int WAVES, int CPW, int PD>
__global__ __launch_bounds__(WAVES * 64) void merge_kernel(MergeParams p) {
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t CHUNK = 128;  // entries per wave load
  constexpr uint32_t B = WAVES * CPW * CHUNK;

  extern __shared__ __attribute__((aligned(16))) uint2 lds[];
  __shared__ Scalars sc;

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t row = blockIdx.x;
  const uint32_t len = static_cast<uint32_t>(p.entries);
  const uint32_t m = (len + B - 1) / B;
  const uint32_t k = static_cast<uint32_t>(p.k);
  const uint32_t B2 = static_cast<uint32_t>(p.slack);

  uint2* const surv0 = lds;
  uint2* const surv1 = lds + k;
  uint2* const app_warm = lds + k;
  uint2* const app_main = lds + 2 * k;
  uint32_t* const hist3 = reinterpret_cast<uint32_t*>(lds + ((2 * k + B2 + B + 1u) & ~1u));  // 16-byte aligned

  for (uint32_t i = tid; i < 3u * kBins; i += NT) hist3[i] = 0;
  if (tid == 0) {
    sc.app_count = 0;
    sc.outpos = 0;
  }
  const uint2* base = p.ws + static_cast<uint64_t>(row) * p.row_entries;  // rows padded to 16 bytes
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint2*>(base), 0, static_cast<int>((len * 8u + 15u) & ~15u), kRsrcWord3);
  BlockOrder ord;
  ord.init(p.seed, row, 0x7FFFFFFFu, m);

  bool accept_all = true;
  uint64_t thr_c = 0, maxc = 0;
  Thr thr{0, 0};
  uint32_t nsurv = 0, cur = 0, napp = 0, hctr = 0;

  u32x4 ring[PD][CPW];
  uint32_t bids[PD];
#pragma unroll
  for (uint32_t d = 0; d < PD; ++d) {
    if (d < m) {
      const uint32_t b = ord.at(d);
      bids[d] = b;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) ring[d][t] = load16(rs, (b * B + (wave + t * WAVES) * CHUNK + lane * 2) * 8u);
    }
  }
  lds_sync();

  for (uint32_t i0 = 0; i0 < m; i0 += PD) {
#pragma unroll
    for (uint32_t d = 0; d < PD; ++d) {
      const uint32_t i = i0 + d;
      if (i >= m) break;
      const uint32_t bid = bids[d];
      u32x4 v[CPW];
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) v[t] = ring[d][t];
      if (i + PD < m) {
        const uint32_t nb = ord.at(i + PD);
        bids[d] = nb;
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t)
          ring[d][t] = load16(rs, (nb * B + (wave + t * WAVES) * CHUNK + lane * 2) * 8u);
      }
      const uint32_t blk_lo = bid * B;
      bool h[CPW][2];
      uint64_t mk[CPW][2];
      uint32_t tot = 0;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) {
        const uint32_t first = blk_lo + (wave + t * WAVES) * CHUNK + lane * 2;
#pragma unroll
        for (uint32_t e = 0; e < 2; ++e) {
          const uint32_t key = v[t][2 * e], idx = v[t][2 * e + 1];
          const bool beats = accept_all || key > thr.key || (key == thr.key && idx < thr.idx);
          h[t][e] = beats && first + e < len;
          mk[t][e] = ballot(h[t][e]);
          tot += popc(mk[t][e]);
        }
      }
      uint32_t pos = 0;
      if (lane == 0) pos = atomicAdd(&sc.app_count, tot);
      pos = uni(pos);
      if (lane == 0) sc.slot[i & 1u][wave] = pos + tot;
      if (tot) {
        uint2* const app = nsurv ? app_main : app_warm;
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
          for (uint32_t e = 0; e < 2; ++e) {
            if (mk[t][e]) {
              const uint32_t q = mbcnt(mk[t][e], pos);
              if (h[t][e]) app[q] = make_uint2(v[t][2 * e], v[t][2 * e + 1]);
              pos += popc(mk[t][e]);
            }
          }
        }
      }
      lds_sync();
      uint32_t cnt = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) cnt = max(cnt, sc.slot[i & 1u][w]);
      napp = cnt;
      if (nsurv + napp >= k + B2) {
        uint2* const sout = nsurv ? (cur ? surv0 : surv1) : surv0;
        const uint2* const sin = cur ? surv1 : surv0;
        compact<DT, WAVES, false>(sin, nsurv, nsurv ? app_main : app_warm, napp, sout, k, sc, hist3, hctr, thr_c,
                                  maxc);
        thr = Thr{static_cast<uint32_t>(thr_c >> 32), ~static_cast<uint32_t>(thr_c)};
        accept_all = false;
        cur = nsurv ? (cur ^ 1u) : 0u;
        nsurv = k;
        napp = 0;
      }
    }
  }
  uint2* const fin = nsurv ? (cur ? surv0 : surv1) : surv0;
  {
    const uint2* const sin = cur ? surv1 : surv0;
    compact<DT, WAVES, false>(sin, nsurv, nsurv ? app_main : app_warm, napp, fin, k, sc, hist3, hctr, thr_c, maxc);
  }
  lds_sync();
  sort_and_store<DT, WAVES>(reinterpret_cast<uint64_t*>(app_main), fin, k, p.out_vals, p.out_idx, row);
}

// --------------------------------------------------------------------------- probes
constexpr uint32_t kProbeThreads = 256;
constexpr uint32_t kProbeUnroll = 4;
constexpr uint32_t kProbeTile = kProbeThreads * 16 * kProbeUnroll;  // bytes per workgroup step

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* src, int64_t vecs, uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads * kProbeUnroll;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads * kProbeUnroll + threadIdx.x; i < vecs;
       i += stride) {
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * kProbeThreads;
      r[u] = j < vecs ? src[j] : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  for (uint32_t o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63u) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (uint32_t w = 0; w < kProbeThreads / 64; ++w) a ^= part[w];
    sink[blockIdx.x] = a;
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(u32x4* dst, const u32x4* src, int64_t vecs) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads * kProbeUnroll;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kProbeThreads * kProbeUnroll + threadIdx.x; i < vecs;
       i += stride) {
    u32x4 r[kProbeUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * kProbeThreads;
      if (j < vecs) r[u] = src[j];
    }
#pragma unroll
    for (uint32_t u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * kProbeThreads;
      if (j < vecs) dst[j] = r[u];
    }
  }
}

// prefetch ring depth: about eight 1 KiB wave chunks in flight per wave
constexpr int ring_depth(int cpw) { return cpw >= 4 ? 2 : (cpw == 2 ? 4 : 8); }

template <int DT, int W, int C>
hipError_t launch_select_shape(const SelectParams& p, int64_t rows, size_t lds, hipStream_t stream) {
  auto kern = select_kernel<DT, W, C, ring_depth(C)>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(rows * p.slices)), dim3(W * 64), lds, stream, p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_select_dt(int shape, const SelectParams& p, int64_t rows, size_t lds, hipStream_t s) {
  switch (shape) {
    case 0: return launch_select_shape<DT, 2, 1>(p, rows, lds, s);
    case 1: return launch_select_shape<DT, 4, 1>(p, rows, lds, s);
    case 2: return launch_select_shape<DT, 4, 2>(p, rows, lds, s);
    case 3: return launch_select_shape<DT, 8, 1>(p, rows, lds, s);
    case 4: return launch_select_shape<DT, 8, 2>(p, rows, lds, s);
    case 5: return launch_select_shape<DT, 4, 4>(p, rows, lds, s);
    case 6: return launch_select_shape<DT, 8, 4>(p, rows, lds, s);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t launch_merge_dt(const MergeParams& p, int64_t rows, size_t lds, hipStream_t stream) {
  constexpr int W = kMergeShape.waves, C = kMergeShape.cpw;
  auto kern = merge_kernel<DT, W, C, ring_depth(C)>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(rows)), dim3(W * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t select_lds_bytes(int k, int block, int slack, int waves) {
  (void)waves;
  return (static_cast<size_t>(2) * k + slack + block + 1) * 8 + 3 * kBins * 4 + sizeof(Scalars);
}

hipError_t launch_select(int dtype, int shape_index, const SelectParams& p, int64_t rows, size_t lds_bytes,
                         hipStream_t stream) {
  const size_t dyn = lds_bytes - sizeof(Scalars);
  return dtype == DS_BF16 ? launch_select_dt<DS_BF16>(shape_index, p, rows, dyn, stream)
                          : launch_select_dt<DS_FP32>(shape_index, p, rows, dyn, stream);
}

hipError_t launch_merge(int dtype, const MergeParams& p, int64_t rows, size_t lds_bytes, hipStream_t stream) {
  const size_t dyn = lds_bytes - sizeof(Scalars);
  return dtype == DS_BF16 ? launch_merge_dt<DS_BF16>(p, rows, dyn, stream)
                          : launch_merge_dt<DS_FP32>(p, rows, dyn, stream);
}

int64_t probe_read_groups(int64_t bytes) {
  int64_t g = (bytes + kProbeTile - 1) / kProbeTile;
  return g < 1 ? 1 : (g > 4096 ? 4096 : g);
}

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t g = probe_read_groups(bytes);
  hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<uint32_t>(g)), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t g = probe_read_groups(bytes);
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<uint32_t>(g)), dim3(kProbeThreads), 0, stream,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), bytes / 16);
  return hipGetLastError();
}

}  // namespace ds
