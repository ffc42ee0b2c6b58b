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
  uint32_t red[kMaxWaves][2];       // per-wave min / max keys
  uint32_t scan[4];                 // bin scan result published by wave 0
  uint32_t lkey[kListCap];          // pivot-bin entries
  uint32_t lidx[kListCap];
  unsigned long long reads;         // counters (stats runs only)
  unsigned long long index_sum;
};

// Candidate buffer in LDS, keys and indices in separate arrays (16-byte aligned, capacity a
// multiple of 4). Entries [0, nsurv) are survivors (keys), [nsurv, n) were appended since the
// last compaction (raw element bits in the select kernel; bf16 in the high half). tkey/tidx
// (k entries) receive the scattered survivors of a compaction.
struct Cand {
  uint32_t* key;
  uint32_t* idx;
  uint32_t* tkey;
  uint32_t* tidx;
};

struct Thr {
  uint32_t key, idx;
};

__device__ __forceinline__ uint64_t comp_of(uint32_t key, uint32_t idx) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~idx);
}

__device__ __forceinline__ uint32_t bitlen32(uint32_t v) { return v ? 32u - static_cast<uint32_t>(__builtin_clz(v)) : 0u; }

__device__ __forceinline__ uint32_t wave_max32(uint32_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t m = 1; m < 64; m <<= 1) v = max(v, xor_lane(v, m, lane));
  return v;
}

__device__ __forceinline__ uint32_t wave_min32(uint32_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t m = 1; m < 64; m <<= 1) v = min(v, xor_lane(v, m, lane));
  return v;
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, uint32_t q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// One wave scans a kBins-bin histogram from the top bin down and finds the bin that holds the
// `need`-th best entry: `above` entries lie in higher bins, `cnt` in that bin.
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
// Reduces the n entries of the candidate buffer to the k best under the composite order
// (key descending, then index ascending). In-loop calls (fin == false) leave the survivors in
// entries [0, k) of the buffer and return the smallest of them as the new threshold
// (tkey, tidx) and the largest key in maxkey; the final call (fin == true) leaves them in
// tkey/tidx (padded with sentinels when n < k).
//
// Search: a kBins-bin histogram of (key - lo) >> shift over a key window [lo, hi] that holds
// every entry locates the bin of the k-th best; while that bin holds more than kListCap
// entries the window shrinks to it and the histogram repeats; a bin that is a single key
// (ties) continues on the indices in [ilo, ihi] (smaller index first). Then the entries
// above the pivot bin are scattered out, the bin's entries are gathered in a short list, and
// the list is ranked to pick the rest and the threshold.
// First call (nsurv == 0): one pass turns raw entries into keys and measures the window.
// Later calls: the window is [threshold key, previous maximum key]; new entries above it fall
// into the top bin ("open" bin, refined over [bin start, true maximum]); the raw -> key step
// is folded into the first histogram pass.
template <int DT, int WAVES, bool RAW>
__device__ void compact(const Cand& c, uint32_t n, uint32_t nsurv, uint32_t k, bool fin, uint32_t ilo,
                        uint32_t ihi, Scalars& sc, uint32_t* hist3, uint32_t& hctr, uint32_t& tkey,
                        uint32_t& tidx, uint32_t& maxkey) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t groups = (n + 3u) / 4u;  // entries are visited four at a time
  auto conv = [](uint32_t raw) { return key_of_raw<DT>(DT == DS_BF16 ? (raw >> 16) : raw); };

  if (n <= k) {  // keep everything (only the final call can get here)
    for (uint32_t i = tid; i < k; i += NT) {
      uint32_t key = 0, id = kSentinelIdx;
      if (i < n) {
        key = c.key[i];
        if (RAW && i >= nsurv) key = conv(key);
        id = c.idx[i];
      }
      c.tkey[i] = key;
      c.tidx[i] = id;
    }
    lds_sync();
    return;
  }

  bool raw_pending = RAW;
  uint32_t lo, hi;
  bool top_open;
  if (nsurv == 0) {
    uint32_t mn = ~0u, mx = 0;
    for (uint32_t g = tid; g < groups; g += NT) {
      uint4 kk = *reinterpret_cast<const uint4*>(c.key + 4 * g);
      if constexpr (RAW) {
        kk.x = conv(kk.x);
        kk.y = conv(kk.y);
        kk.z = conv(kk.z);
        kk.w = conv(kk.w);
        *reinterpret_cast<uint4*>(c.key + 4 * g) = kk;
      }
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) {
        if (4 * g + q < n) {
          mn = min(mn, u4get(kk, q));
          mx = max(mx, u4get(kk, q));
        }
      }
    }
    mn = wave_min32(mn, lane);
    mx = wave_max32(mx, lane);
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
    lo = ~0u;
    hi = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      lo = min(lo, sc.red[w][0]);
      hi = max(hi, sc.red[w][1]);
    }
    top_open = false;
    raw_pending = false;
  } else {
    lo = tkey;  // every entry ranks at or above the threshold
    hi = maxkey;
    top_open = true;
    if (tid == 0) {  // every wave passed the block barrier after its appends
      sc.app_count = 0;
      sc.outpos = 0;
      sc.listpos = 0;
    }
  }

  // histogram passes
  uint32_t need = k, above_total = 0, cnt = 0, seen_max = 0;
  uint32_t plo = lo, phi = hi;  // key window of the pivot
  bool tie = false;             // pivot window is a single key: continue on indices
  uint32_t pkey = 0, iplo = ilo, iphi = ihi;
  for (;;) {
    const uint32_t range = tie ? iphi - iplo : phi - plo;
    const uint32_t shift = bitlen32(range) > 9 ? bitlen32(range) - 9 : 0;
    uint32_t* h = hist3 + kBins * (hctr % 3u);
    uint32_t* hn = hist3 + kBins * ((hctr + 1u) % 3u);
    for (uint32_t b = tid; b < kBins; b += NT) hn[b] = 0;
    uint32_t mx = 0;
    for (uint32_t g = tid; g < groups; g += NT) {
      uint4 kk = *reinterpret_cast<const uint4*>(c.key + 4 * g);
      if (raw_pending && 4 * g + 3 >= nsurv) {
        if (4 * g + 0 >= nsurv) kk.x = conv(kk.x);
        if (4 * g + 1 >= nsurv) kk.y = conv(kk.y);
        if (4 * g + 2 >= nsurv) kk.z = conv(kk.z);
        kk.w = conv(kk.w);
        *reinterpret_cast<uint4*>(c.key + 4 * g) = kk;
      }
      if (!tie) {
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          const uint32_t key = u4get(kk, q);
          if (4 * g + q < n) {
            mx = max(mx, key);
            if (key >= plo && (key <= phi || top_open)) atomicAdd(&h[(min(key, phi) - plo) >> shift], 1u);
          }
        }
      } else {
        const uint4 ii = *reinterpret_cast<const uint4*>(c.idx + 4 * g);
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          const uint32_t key = u4get(kk, q), id = u4get(ii, q);
          if (4 * g + q < n) {
            mx = max(mx, key);
            if (key == pkey && id >= iplo && id <= iphi) atomicAdd(&h[kBins - 1u - ((id - iplo) >> shift)], 1u);
          }
        }
      }
    }
    raw_pending = false;
    mx = wave_max32(mx, lane);
    if (lane == 0) sc.red[wave][1] = mx;
    lds_sync();
    ++hctr;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) seen_max = max(seen_max, sc.red[w][1]);
    uint32_t bin, above;
    if constexpr (WAVES > 4) {  // one wave scans and publishes the result
      if (wave == 0) {
        scan_select(h, need, lane, bin, above, cnt);
        if (lane == 0) {
          sc.scan[0] = bin;
          sc.scan[1] = above;
          sc.scan[2] = cnt;
        }
      }
      lds_sync();
      bin = sc.scan[0];
      above = sc.scan[1];
      cnt = sc.scan[2];
    } else {
      scan_select(h, need, lane, bin, above, cnt);
    }
    need -= above;
    above_total += above;
    if (!tie) {
      const uint32_t nlo = plo + (bin << shift);
      const bool open_bin = top_open && bin == ((phi - plo) >> shift);
      const uint64_t nhi64 = static_cast<uint64_t>(plo) + ((static_cast<uint64_t>(bin) + 1u) << shift) - 1u;
      const uint32_t nhi = nhi64 > phi ? phi : static_cast<uint32_t>(nhi64);
      plo = nlo;
      phi = open_bin ? seen_max : nhi;
      top_open = false;
      if (cnt <= kListCap) break;
      if (shift == 0 && !open_bin) {  // one key holds more than kListCap entries
        tie = true;
        pkey = plo;
      }
    } else {
      const uint32_t nlo = iplo + ((kBins - 1u - bin) << shift);
      const uint64_t nhi64 = static_cast<uint64_t>(nlo) + (1ull << shift) - 1u;
      iphi = nhi64 > iphi ? iphi : static_cast<uint32_t>(nhi64);
      iplo = nlo;
      if (cnt <= kListCap || shift == 0) break;
    }
  }
  cnt = cnt < kListCap ? cnt : kListCap;  // more only if (key, index) pairs repeat

  // scatter: entries above the pivot window go out, the window's entries to the list
  const uint32_t iters = (groups + NT - 1) / NT;
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t g = it * NT + tid;
    uint4 kk = make_uint4(0, 0, 0, 0), ii = make_uint4(0, 0, 0, 0);
    if (g < groups) {
      kk = *reinterpret_cast<const uint4*>(c.key + 4 * g);
      ii = *reinterpret_cast<const uint4*>(c.idx + 4 * g);
    }
    bool up[4], mid[4];
    uint64_t bu[4], bm[4];
    uint32_t nu = 0, nm = 0;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
      const uint32_t key = u4get(kk, q), id = u4get(ii, q);
      const bool valid = g < groups && 4 * g + q < n;
      if (!tie) {
        up[q] = valid && key > phi;
        mid[q] = valid && key >= plo && key <= phi;
      } else {
        up[q] = valid && (key > pkey || (key == pkey && id < iplo));
        mid[q] = valid && key == pkey && id >= iplo && id <= iphi;
      }
      bu[q] = ballot(up[q]);
      bm[q] = ballot(mid[q]);
      nu += popc(bu[q]);
      nm += popc(bm[q]);
    }
    if (nu | nm) {
      uint32_t b0 = 0, b1 = 0;
      if (lane == 0) {
        if (nu) b0 = atomicAdd(&sc.outpos, nu);
        if (nm) b1 = atomicAdd(&sc.listpos, nm);
      }
      b0 = uni(b0);
      b1 = uni(b1);
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) {
        if (up[q]) {
          const uint32_t at = mbcnt(bu[q], b0);
          if (at < k) {
            c.tkey[at] = u4get(kk, q);
            c.tidx[at] = u4get(ii, q);
          }
        }
        if (mid[q]) {
          const uint32_t at = mbcnt(bm[q], b1);
          if (at < kListCap) {
            sc.lkey[at] = u4get(kk, q);
            sc.lidx[at] = u4get(ii, q);
          }
        }
        b0 += popc(bu[q]);
        b1 += popc(bm[q]);
      }
    }
  }
  lds_sync();

  // every wave ranks the short list: the `need` best of its cnt entries are kept
  const bool have = lane < cnt;
  const uint32_t lk = have ? sc.lkey[lane] : 0u, li = have ? sc.lidx[lane] : kSentinelIdx;
  const uint64_t mine = comp_of(lk, li);
  uint32_t rank = 0;
  for (uint32_t m = 0; m < cnt; ++m) rank += readlane64(mine, m) > mine ? 1u : 0u;
  const bool keep = have && rank < need;
  const uint64_t piv = ballot(have && rank == need - 1u);
  const uint32_t pl = piv ? static_cast<uint32_t>(__builtin_ctzll(piv)) : 0u;
  tkey = __builtin_amdgcn_readlane(lk, pl);
  tidx = __builtin_amdgcn_readlane(li, pl);
  maxkey = seen_max;
  if (!fin) {
    for (uint32_t i = tid; i < above_total && i < k; i += NT) {
      c.key[i] = c.tkey[i];
      c.idx[i] = c.tidx[i];
    }
    if (wave == 0 && keep) {
      c.key[above_total + rank] = lk;
      c.idx[above_total + rank] = li;
    }
  } else {
    if (wave == 0 && keep) {
      c.tkey[above_total + rank] = lk;
      c.tidx[above_total + rank] = li;
    }
    lds_sync();
  }
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

template <int DT>
__device__ __forceinline__ void store_out(void* out_vals, int32_t* out_idx, uint64_t at, uint64_t c) {
  const uint32_t key = static_cast<uint32_t>(c >> 32), id = ~static_cast<uint32_t>(c);
  if (out_vals) {
    if constexpr (DT == DS_BF16)
      static_cast<uint16_t*>(out_vals)[at] = static_cast<uint16_t>(raw_of_key<DT>(key));
    else
      static_cast<uint32_t*>(out_vals)[at] = raw_of_key<DT>(key);
  }
  if (out_idx) out_idx[at] = static_cast<int32_t>(id);
}

// Sort the k entries of (fkey, fidx) (padded with sentinels to NT*E) best first and store the
// first k of them.
template <int DT, int WAVES, int E>
__device__ void sort_store_e(const uint32_t* fkey, const uint32_t* fidx, uint64_t* xbuf, uint32_t k,
                             void* out_vals, int32_t* out_idx, uint64_t row) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  uint64_t v[E];
#pragma unroll
  for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
    const uint32_t e = tid * E + j;
    v[j] = e < k ? comp_of(fkey[e], fidx[e]) : 0ull;
  }
  lds_sync();  // xbuf may overlap memory other threads are still reading above
  bitonic_stages<WAVES, E, 2, 1>(v, xbuf, tid, lane);
#pragma unroll
  for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
    const uint32_t e = tid * E + j;
    if (e < k) store_out<DT>(out_vals, out_idx, row * k + e, v[j]);
  }
}

// Bitonic sort in LDS (one barrier per stage) for k above four entries per thread: sorts cap
// (a power of two >= k) composites in `xbuf`, best first, and stores the first k.
template <int DT, int WAVES>
__device__ void sort_store_lds(const uint32_t* fkey, const uint32_t* fidx, uint64_t* xbuf, uint32_t k,
                               void* out_vals, int32_t* out_idx, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x;
  uint32_t cap = 1;
  while (cap < k) cap <<= 1;
  // xbuf may overlap (fkey, fidx): read everything into registers first, in two halves
  for (uint32_t base = 0; base < cap; base += NT * 8) {
    uint64_t tmp[8];
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
      const uint32_t i = base + j * NT + tid;
      tmp[j] = i < k ? comp_of(fkey[i], fidx[i]) : 0ull;
    }
    lds_sync();
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
      const uint32_t i = base + j * NT + tid;
      if (i < cap) xbuf[i] = tmp[j];
    }
    lds_sync();
  }
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
  for (uint32_t i = tid; i < k; i += NT) store_out<DT>(out_vals, out_idx, row * k + i, xbuf[i]);
}

// `xbuf` needs max(NT, pow2 >= k) 64-bit slots; (fkey, fidx) must be visible to every thread.
template <int DT, int WAVES>
__device__ void sort_and_store(uint64_t* xbuf, const uint32_t* fkey, const uint32_t* fidx, uint32_t k,
                               void* out_vals, int32_t* out_idx, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  if (k <= NT)
    sort_store_e<DT, WAVES, 1>(fkey, fidx, xbuf, k, out_vals, out_idx, row);
  else if (k <= 2 * NT)
    sort_store_e<DT, WAVES, 2>(fkey, fidx, xbuf, k, out_vals, out_idx, row);
  else if (k <= 4 * NT)
    sort_store_e<DT, WAVES, 4>(fkey, fidx, xbuf, k, out_vals, out_idx, row);
  else
    sort_store_lds<DT, WAVES>(fkey, fidx, xbuf, k, out_vals, out_idx, row);
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

// LDS layout shared by both kernels (32-bit words): key[cap] idx[cap] tkey[k4] tidx[k4]
// hist[3*kBins], with cap = k + B2 + B and k4 = k, both rounded up to multiples of 4.
__host__ __device__ constexpr uint32_t round4(uint32_t v) { return (v + 3u) & ~3u; }

__device__ __forceinline__ Cand cand_layout(uint32_t* lds, uint32_t k, uint32_t B2, uint32_t B, uint32_t*& hist3) {
  const uint32_t cap = round4(k + B2 + B), k4 = round4(k);
  Cand c;
  c.key = lds;
  c.idx = lds + cap;
  c.tkey = lds + 2 * cap;
  c.tidx = lds + 2 * cap + k4;
  hist3 = lds + 2 * cap + 2 * k4;
  return c;
}

// --------------------------------------------------------------------------- select kernel
// Byte offset past every buffer range: a load there returns zeros and reads no memory.
constexpr uint32_t kNoLoad = 0x7FFFFFF0u;

template <int DT, int WAVES, int CPW, int PD>
__global__ __launch_bounds__(WAVES * 64) void select_kernel(SelectParams p) {
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t EB = DT == DS_BF16 ? 2 : 4;
  constexpr uint32_t VEC = 16 / EB;
  constexpr uint32_t CHUNK = 64 * VEC;
  constexpr uint32_t B = WAVES * CPW * CHUNK;

  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
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

  uint32_t* hist3;
  const Cand c = cand_layout(lds, k, B2, B, hist3);

  for (uint32_t i = tid; i < 3u * kBins; i += NT) hist3[i] = 0;
  if (tid == 0) {
    sc.app_count = 0;
    sc.outpos = 0;
    sc.listpos = 0;
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
  uint32_t mode = 0, thr_s = 0, thr_n = 0;
  uint32_t t_key = 0, t_idx = 0, maxkey = 0;
  uint32_t nsurv = 0, napp = 0, hctr = 0;
  // counters (thread-uniform; used when stats are requested)
  uint64_t st_a = 0, st_r = 0, st_w = 0, st_max = 0, st_mono = 1, my_reads = 0, my_jsum = 0;
  uint64_t t_start = stats ? wall_clock64() : 0, t_compact = 0, t_sync = 0, t_mark = 0;

  // Two-stage pipeline: at the top of block i the wave takes block i's chunks (loaded during
  // block i-1) and at once issues the loads of block i+1, which stay in flight through the
  // filter, the barrier and any compaction. Past the last block the loads go to kNoLoad.
  u32x4 next[CPW];
  uint32_t next_bid = ord.at(0);
#pragma unroll
  for (uint32_t t = 0; t < CPW; ++t) next[t] = load16(rs, (next_bid * B + (wave + t * WAVES) * CHUNK + lane * VEC) * EB);
  lds_sync();

  for (uint32_t i = 0; i < m; ++i) {
    u32x4 cur[CPW];
#pragma unroll
    for (uint32_t t = 0; t < CPW; ++t) cur[t] = next[t];
    const uint32_t bid = next_bid;
    {
      const bool live = i + 1 < m;
      next_bid = live ? ord.at(i + 1) : 0u;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t)
        next[t] = load16(rs, live ? (next_bid * B + (wave + t * WAVES) * CHUNK + lane * VEC) * EB : kNoLoad);
    }
    const uint32_t blk_lo = bid * B;
    const bool strict = slice_lo + blk_lo > t_idx;
    const uint32_t thr = strict ? thr_s : thr_n;

    // ---- filter: scores (bf16 elements in the high half) and hit masks
    uint32_t s[CPW][VEC];
    bool h[CPW][VEC];
#pragma unroll
    for (uint32_t t = 0; t < CPW; ++t) {
      if constexpr (DT == DS_BF16) {
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          s[t][2 * q] = cur[t][q] << 16;
          s[t][2 * q + 1] = cur[t][q];
        }
      } else {
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) s[t][q] = cur[t][q];
      }
    }
    if (mode == 1) {
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t)
#pragma unroll
        for (uint32_t e = 0; e < VEC; ++e) h[t][e] = static_cast<int32_t>(s[t][e]) > static_cast<int32_t>(thr);
    } else if (mode == 2) {
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t)
#pragma unroll
        for (uint32_t e = 0; e < VEC; ++e) h[t][e] = s[t][e] < thr;
    } else {
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t)
#pragma unroll
        for (uint32_t e = 0; e < VEC; ++e) h[t][e] = true;
    }
    uint64_t mk[CPW][VEC];
    uint32_t tot = 0;
#pragma unroll
    for (uint32_t t = 0; t < CPW; ++t) {
      const uint32_t off = blk_lo + (wave + t * WAVES) * CHUNK;
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
      pos += nsurv;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) {
        const uint32_t jl = slice_lo + blk_lo + (wave + t * WAVES) * CHUNK + lane * VEC;
#pragma unroll
        for (uint32_t e = 0; e < VEC; ++e) {
          if (mk[t][e]) {
            const uint32_t q = mbcnt(mk[t][e], pos);
            if (h[t][e]) {
              c.key[q] = s[t][e];
              c.idx[q] = jl + e;
            }
            pos += popc(mk[t][e]);
          }
        }
      }
    }
    if (stats) t_mark = wall_clock64();
    lds_sync();
    if (stats) t_sync += wall_clock64() - t_mark;

    // ---- compaction test after the whole block
    uint32_t cnt = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) cnt = max(cnt, sc.slot[i & 1u][w]);
    napp = cnt;
    st_max = max(st_max, static_cast<uint64_t>(nsurv + napp));
    if (nsurv + napp >= k + B2) {
      const uint64_t prev_c = comp_of(t_key, t_idx);
      const bool first = nsurv == 0;
      if (stats) t_mark = wall_clock64();
      compact<DT, WAVES, true>(c, nsurv + napp, nsurv, k, false, slice_lo, slice_lo + len - 1u, sc, hist3, hctr,
                               t_key, t_idx, maxkey);
      if (stats) t_compact += wall_clock64() - t_mark;
      st_a += napp;
      st_w += nsurv + napp;
      st_r += 1;
      if (!first && comp_of(t_key, t_idx) < prev_c) st_mono = 0;
      nsurv = k;
      napp = 0;
      filter_thresholds<DT>(Thr{t_key, t_idx}, mode, thr_s, thr_n);
    }
  }

  // ---- final compaction: survivors to (tkey, tidx)
  const uint64_t t_final0 = stats ? wall_clock64() : 0;
  compact<DT, WAVES, true>(c, nsurv + napp, nsurv, k, true, slice_lo, slice_lo + len - 1u, sc, hist3, hctr, t_key,
                           t_idx, maxkey);
  st_a += napp;
  st_w += nsurv + napp;

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
      o->t_compact_ns = t_compact * 10;
      o->t_sync_ns = t_sync * 10;
      o->reserved = 0;
    }
  }

  if (p.slices == 1) {
    sort_and_store<DT, WAVES>(reinterpret_cast<uint64_t*>(c.key), c.tkey, c.tidx, k, p.out_vals, p.out_idx, row);
  } else {
    uint2* const dst = p.ws + static_cast<uint64_t>(row) * p.ws_row_entries + static_cast<uint64_t>(slice) * k;
    for (uint32_t i = tid; i < k; i += NT) dst[i] = make_uint2(c.tkey[i], c.tidx[i]);
  }
  if (stats && tid == 0) {
    const uint64_t t_end = wall_clock64();
    p.stats[blockIdx.x].t_total_ns = (t_end - t_start) * 10;
    p.stats[blockIdx.x].t_final_ns = (t_end - t_final0) * 10;
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

  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ Scalars sc;

  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t row = blockIdx.x;
  const uint32_t len = static_cast<uint32_t>(p.entries);
  const uint32_t m = (len + B - 1) / B;
  const uint32_t k = static_cast<uint32_t>(p.k);
  const uint32_t B2 = static_cast<uint32_t>(p.slack);

  uint32_t* hist3;
  const Cand c = cand_layout(lds, k, B2, B, hist3);
  for (uint32_t i = tid; i < 3u * kBins; i += NT) hist3[i] = 0;
  if (tid == 0) {
    sc.app_count = 0;
    sc.outpos = 0;
    sc.listpos = 0;
  }
  const uint2* base = p.ws + static_cast<uint64_t>(row) * p.row_entries;  // rows padded to 16 bytes
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint2*>(base), 0, static_cast<int>((len * 8u + 15u) & ~15u), kRsrcWord3);
  BlockOrder ord;
  ord.init(p.seed, row, 0x7FFFFFFFu, m);

  bool accept_all = true;
  uint32_t t_key = 0, t_idx = 0, maxkey = 0;
  uint32_t nsurv = 0, napp = 0, hctr = 0;

  u32x4 next[CPW];
  uint32_t next_bid = ord.at(0);
#pragma unroll
  for (uint32_t t = 0; t < CPW; ++t) next[t] = load16(rs, (next_bid * B + (wave + t * WAVES) * CHUNK + lane * 2) * 8u);
  lds_sync();

  for (uint32_t i = 0; i < m; ++i) {
    u32x4 v[CPW];
#pragma unroll
    for (uint32_t t = 0; t < CPW; ++t) v[t] = next[t];
    const uint32_t bid = next_bid;
    {
      const bool live = i + 1 < m;
      next_bid = live ? ord.at(i + 1) : 0u;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t)
        next[t] = load16(rs, live ? (next_bid * B + (wave + t * WAVES) * CHUNK + lane * 2) * 8u : kNoLoad);
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
        const bool beats = accept_all || key > t_key || (key == t_key && idx < t_idx);
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
      pos += nsurv;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
        for (uint32_t e = 0; e < 2; ++e) {
          if (mk[t][e]) {
            const uint32_t q = mbcnt(mk[t][e], pos);
            if (h[t][e]) {
              c.key[q] = v[t][2 * e];
              c.idx[q] = v[t][2 * e + 1];
            }
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
      compact<DT, WAVES, false>(c, nsurv + napp, nsurv, k, false, 0u, static_cast<uint32_t>(p.n - 1), sc, hist3,
                                hctr, t_key, t_idx, maxkey);
      accept_all = false;
      nsurv = k;
      napp = 0;
    }
  }
  compact<DT, WAVES, false>(c, nsurv + napp, nsurv, k, true, 0u, static_cast<uint32_t>(p.n - 1), sc, hist3, hctr,
                            t_key, t_idx, maxkey);
  sort_and_store<DT, WAVES>(reinterpret_cast<uint64_t*>(c.key), c.tkey, c.tidx, k, p.out_vals, p.out_idx, row);
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
constexpr int ring_depth(int cpw) { return cpw > 0 ? 1 : 1; }  // one block in flight per wave (two-stage pipeline)

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
    case 7: return launch_select_shape<DT, 16, 1>(p, rows, lds, s);
    case 8: return launch_select_shape<DT, 16, 2>(p, rows, lds, s);
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
  const size_t cap = round4(static_cast<uint32_t>(k + slack + block)), k4 = round4(static_cast<uint32_t>(k));
  return (2 * cap + 2 * k4 + 3 * kBins) * 4 + sizeof(Scalars);
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
