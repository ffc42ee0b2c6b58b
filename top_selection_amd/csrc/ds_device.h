#pragma once
// DeepSelect row-wise top-k: HIP device code for gfx950 (CDNA4, 64-lane waves), shared by the
// translation units that instantiate and launch it (ds_select.hip, ds_merge.hip).
//
// Method (DeepSelect design note, "Algorithm"): a threshold T, blocks of B elements read
// once in a random order independent of the data, a filter that appends every element
// beating T to an on-chip candidate buffer, a radix-select compaction back to k entries
// whenever the buffer reaches k + B2 (which also raises T to the smallest survivor), and a
// final compaction. The split-row path (design note, "Implementation", cluster paragraph)
// runs the same method on slices of a row and merges the slices' survivors: each slice
// stores a sorted list, and a list-merge kernel places entries by rank, in levels of up to
// 16 lists (or, when asked, the method runs again over all survivors).
//
// Order used everywhere: an element is the pair (value, index); larger value first,
// +0 before -0, then smaller index first. On the device an element's value is replaced
// by an order-preserving unsigned "key" (tutorial chapter section 4.6: positive values get
// their sign bit flipped, negative values all bits inverted), and a pair by the 64-bit
// composite (key << 32) | ~index, so every comparison is an integer comparison.
//
// MI355X mapping:
//  * one workgroup (2-16 waves) per (row, slice); every lane streams 16-byte raw buffer
//    loads (1 KiB per wave per chunk). Each wave keeps D blocks in flight (D buffers of
//    registers): block i+D is loaded into the registers of block i as soon as block i has
//    been filtered, so loads stay in flight through the block barrier and any compaction.
//    The random order is over groups of G consecutive blocks (a table in LDS, computed once
//    per workgroup), so consecutive loads are in flight together;
//  * the first whole block may set a presampled threshold (a lower bound of its k-th
//    element, from the lanes' maxima) instead of accepting everything;
//  * the filter compares raw bit patterns against a per-block integer threshold; hit masks
//    are 64-lane SGPR masks, positions come from mbcnt, and one LDS atomic per wave and chunk
//    reserves buffer space. Hits are stored raw; the compaction's first pass turns them
//    into keys;
//  * barriers are LDS-only (s_barrier with workgroup/local fences), so in-flight global
//    loads are never drained by a barrier;
//  * the compaction is an LDS radix select with 2048-bin histograms: the first pass bins
//    values linearly over [T, previous maximum] (floats crowd into few key bins), later
//    passes bin keys or indices. All waves count, one wave scans the bins and publishes the
//    pivot bin, and in the usual case one pass leaves at most 64 pivot-bin entries, which
//    one wave ranks with lane reads. Survivors alternate between two k-entry sets, so
//    nothing is copied back; appends always go to the region after the survivor set A. The
//    final compaction can write its survivors sorted (a counting sort over its value bins).
#include <atomic>
#include <type_traits>

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

// Work item of workgroup `wg` when each unit (a row) has `per` workgroups and `units` units:
// the units are dealt to the eight XCDs (workgroup i runs on XCD i mod 8) so that all
// workgroups of a unit run on one XCD and share its L2; units past the last multiple of 8
// follow in plain order. Returns the unit and the workgroup's index within it.
// a / d and a % d for a uniform d >= 1: a shift and a mask when d is a power of two (the usual
// slice counts), else the division
__device__ __forceinline__ void divmod_uniform(uint32_t a, uint32_t d, uint32_t& q, uint32_t& r) {
  if ((d & (d - 1u)) == 0u) {
    q = a >> __builtin_ctz(d);
    r = a & (d - 1u);
  } else {
    q = a / d;
    r = a - q * d;
  }
}

__device__ __forceinline__ void xcd_unit(uint32_t wg, uint32_t per, uint32_t units, uint32_t& unit, uint32_t& sub) {
  const uint32_t dealt = (units & ~7u) * per;
  uint32_t q;
  if (wg < dealt) {
    divmod_uniform(wg >> 3, per, q, sub);
    unit = (wg & 7u) + 8u * q;
  } else {
    divmod_uniform(wg - dealt, per, q, sub);
    unit = (units & ~7u) + q;
  }
}

// The same LDS location as an LDS-address-space pointer: accesses through it are always LDS
// instructions (a generic pointer the compiler cannot trace becomes a flat access, which also
// counts as an outstanding global access and makes the compiler wait for every global load).
template <class T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(T* p) {
  return (__attribute__((address_space(3))) T*)p;
}

// LDS byte addresses: a word's address, and the word at an address.
__device__ __forceinline__ uint32_t lds_addr(const uint32_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(const_cast<uint32_t*>(p))));
}
__device__ __forceinline__ __attribute__((address_space(3))) uint32_t* lds_at(uint32_t a) {
  return reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(static_cast<uintptr_t>(a));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t m, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), base));
}

__device__ __forceinline__ uint32_t popc(uint64_t m) { return static_cast<uint32_t>(__popcll(m)); }

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Value held by lane (lane ^ m), m a power of two below 64. Lane mappings (checked on
// gfx950): quad_perm 0xB1 / 0x4E swap neighbours at distance 1 / 2, row_shl:4 / row_shr:4
// bring the lane four above / below within a 16-lane row, row_ror:8 swaps the halves of a
// row, and the permlane16/32 swaps exchange 16-lane rows / 32-lane halves.
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, uint32_t m, uint32_t lane) {
  switch (m) {
    case 1: return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);
    case 4: {
      const uint32_t up = __builtin_amdgcn_update_dpp(0u, v, 0x104, 0xF, 0xF, false);
      const uint32_t dn = __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);
      return (lane & 4u) ? dn : up;
    }
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

// Maximum over the 64 lanes (the same row shifts and broadcasts as the scan, then lane 63).
__device__ __forceinline__ uint32_t wave_max32(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false)));
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ uint32_t wave_min32(uint32_t x) {
  x = min(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, x, 0x111, 0xF, 0xF, false)));
  x = min(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, x, 0x112, 0xF, 0xF, false)));
  x = min(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, x, 0x114, 0xF, 0xF, false)));
  x = min(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, x, 0x118, 0xF, 0xF, false)));
  x = min(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, x, 0x142, 0xA, 0xF, false)));
  x = min(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(~0u, x, 0x143, 0xC, 0xF, false)));
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ uint32_t u4get(const uint4& v, uint32_t q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

__device__ __forceinline__ uint32_t bitlen32(uint32_t v) {
  return v ? 32u - static_cast<uint32_t>(__builtin_clz(v)) : 0u;
}

constexpr uint32_t kLogBins = 11;
constexpr uint32_t kBins = 1u << kLogBins;  // histogram bins of one radix pass

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

// Order-preserving key of a streamed score without branches (bf16: the element in bits 16-31,
// as the filter holds it).
template <int DT>
__device__ __forceinline__ uint32_t key_of_score(uint32_t s) {
  if constexpr (DT == DS_BF16) {
    const uint32_t r = s >> 16;
    return (r ^ (static_cast<uint32_t>(static_cast<int32_t>(s) >> 31) | 0x8000u)) & 0xFFFFu;
  } else {
    return s ^ (static_cast<uint32_t>(static_cast<int32_t>(s) >> 31) | 0x80000000u);
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

__device__ __forceinline__ uint64_t comp_of(uint32_t key, uint32_t idx) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~idx);
}

// Key of +infinity: keys above it are NaN patterns, which never occur.
template <int DT>
constexpr uint32_t key_of_inf() {
  return DT == DS_BF16 ? 0xFF80u : 0xFF800000u;
}

template <int DT>
__device__ __forceinline__ float value_of_key(uint32_t key) {
  if constexpr (DT == DS_BF16)
    return __uint_as_float(raw_of_key<DT>(key) << 16);
  else
    return __uint_as_float(raw_of_key<DT>(key));
}

// Value-space bins: bin(v) = clamp((v - lo) * scale, 0, kBins - 1), truncated, for a window
// [lo, hi] with scale = kBins times the hardware reciprocal of (hi - lo). Any positive scale
// serves: each step is a deterministic fp32 operation (no contraction), so the bin is a
// non-decreasing function of the key and every thread that evaluates it gets the same bin;
// values above hi land in the top bin.
struct VBins {
  float lo, scale;
};

template <int DT>
__device__ __forceinline__ uint32_t vbin(uint32_t key, const VBins& vb) {
#pragma clang fp contract(off)
  const float t = (value_of_key<DT>(key) - vb.lo) * vb.scale;
  return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(t, 0.0f, static_cast<float>(kBins - 1u)));
}

// Window [lo, hi] from two keys; false when value bins cannot be used (an infinite bound or
// span, an empty span, or a scale that overflows).
template <int DT>
__device__ __forceinline__ bool vbins_of(uint32_t klo, uint32_t khi, VBins& vb) {
  const float lo = value_of_key<DT>(klo), hi = value_of_key<DT>(khi);
  const float span = hi - lo;
  vb.lo = lo;
  vb.scale = static_cast<float>(kBins) * __builtin_amdgcn_rcpf(span);
  return __builtin_isfinite(lo) && __builtin_isfinite(hi) && span > 0.0f && __builtin_isfinite(span) &&
         __builtin_isfinite(vb.scale) && vb.scale > 0.0f;
}

// Smallest key K in [klo, kmax] with vbin(K) >= b, or kmax + 1 if there is none: a 64-way
// search by one wave (each round the lanes probe 64 evenly spaced keys).
template <int DT>
__device__ __forceinline__ uint64_t vbin_first_key(uint32_t b, uint32_t klo, uint32_t kmax, const VBins& vb,
                                                   uint32_t lane) {
  uint64_t lo = klo, cnt = static_cast<uint64_t>(kmax) - klo + 1u;  // the answer lies in [lo, lo + cnt]
  while (cnt > 0) {
    const uint64_t step = (cnt + 63u) / 64u;
    const uint64_t off = lane * step;
    const bool probe = off < cnt;
    const bool ok = probe && vbin<DT>(static_cast<uint32_t>(lo + off), vb) >= b;
    const uint32_t j = popc(ballot(probe && !ok));  // the failing probes are a prefix
    if (j == 0) break;
    const uint64_t nlo = lo + (j - 1u) * step + 1u;
    const uint64_t hi_j = lo + j * step, end = lo + cnt;
    cnt = (hi_j < end ? hi_j : end) - nlo;
    lo = nlo;
  }
  return lo;
}

// --------------------------------------------------------------------------- block order
// Keyed Feistel bijection on [0, 2^b) (b the smallest even width >= 2 with 2^b >= m),
// four rounds with the lowbias32 integer hash as round function, restricted to [0, m)
// by cycle walking. Round key r is the low half of the splitmix64 finaliser of
// hs ^ (row << 33 | slice << 2 | r), hs = mix64(seed) (one value per call, mixed on the host):
// distinct (row, slice, r) give distinct inputs to a bijection. The walk ends because the
// permutation's cycle through i returns to i < m.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// A copy of a uniform value in a vector register: arithmetic on it runs in the vector units.
// The CU's waves share one scalar unit, so uniform set-up arithmetic that every wave repeats
// (the block order's keys, the first block ids) is cheaper spread over the SIMDs.
__device__ __forceinline__ uint32_t to_vgpr(uint32_t s) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
  return v;
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

  // hs: the call's mixed seed, mix64(seed), computed once on the host
  __device__ __forceinline__ void init(uint64_t hs, uint32_t row, uint32_t slice, uint32_t m_) {
    // lane l derives key l & 3 in vector registers; the four keys are then read back
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const uint64_t vhs = (static_cast<uint64_t>(to_vgpr(static_cast<uint32_t>(hs >> 32))) << 32) |
                         to_vgpr(static_cast<uint32_t>(hs));
    const uint64_t tag = (static_cast<uint64_t>(to_vgpr(row)) << 33) | (static_cast<uint64_t>(slice) << 2) | (lane & 3u);
    const uint32_t mine = static_cast<uint32_t>(mix64(vhs ^ tag));
#pragma unroll
    for (int r = 0; r < 4; ++r) key[r] = __builtin_amdgcn_readlane(mine, r);
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
constexpr uint32_t kPer = kBins / 64;       // bins per lane in the bin scan
constexpr uint32_t kListCap = 64;           // pivot-bin entries ranked with lane reads
constexpr uint32_t kOrdCap = 1024;          // block-order table entries (longer streams compute it)

struct Scalars {
  uint32_t len;                // entries appended since the last compaction
  uint32_t done;               // waves whose stream has ended (free-running schedule)
  uint32_t outpos;             // scatter cursor of the running compaction
  uint32_t listpos;            // pivot-list cursor of the running compaction
  uint32_t pub[6];             // bin scan result: bin, entries above it, entries in it, max key,
                               // and the key bounds of a value-space bin
  uint32_t red[kMaxWaves];     // per-wave maximum keys
  uint32_t rmin[kMaxWaves];    // per-wave smallest / largest key appended before the first
  uint32_t rmax[kMaxWaves];    // compaction
  uint32_t lkey[kListCap];     // pivot-bin entries
  uint32_t lidx[kListCap];
  uint32_t shr[2];             // the row's shared threshold as read by thread 0 (low, high word)
  uint32_t big;                // one-pass final sort: a bin too full for it (falls back)
  // counters (stats runs only; thread 0 keeps them): appended A, compactions R, work W,
  // largest buffer, threshold monotone, compaction time, block barrier time, start of the
  // final compaction, elements read and the sum of their indices
  unsigned long long st_a, st_r, st_w, st_max, st_mono, st_tc, st_ts, st_tf, reads, index_sum;
  uint32_t st_p;  // histogram passes (counted in every run; reported in stats runs)
};

__host__ __device__ constexpr uint32_t round4(uint32_t v) { return (v + 3u) & ~3u; }

// Candidate buffer in LDS (32-bit words, every array 16-byte aligned), k4 = round4(k),
// pc = round4(B2 + B):
//   ck[k4 + pc + 64], ci[...] keys / indices: survivor set A in [0, k4), appended entries
//                             from k4 on (before the first compaction appends start at 0,
//                             so k + B2 + B entries fit), then 64 per-lane dummy slots
//   bk[k4], bi[k4]            survivor set B
//   hist[2 * kBins]           two histograms, used alternately
//   ordt[kOrdCap]             the block order (block id of the i-th block read)
// After the final compaction the append region (ck + k4, ci + k4: pc >= pow2(k) words
// each) is the sort's exchange buffer.
// Per-lane dummy slots after the append region of ck and ci: a lane whose element does not
// hit writes there, so the append needs no exec-mask changes.
constexpr uint32_t kDummySlots = 64;

struct Lay {
  uint32_t *ck, *ci, *bk, *bi, *hist, *ordt;
  uint32_t k4, pc, dummy;
};

__device__ __forceinline__ Lay lay_of(uint32_t* lds, uint32_t k, uint32_t B2, uint32_t B) {
  Lay l;
  l.k4 = round4(k);
  l.pc = round4(B2 + B);
  l.dummy = l.k4 + l.pc;
  l.ck = lds;
  l.ci = lds + (l.k4 + l.pc + kDummySlots);
  l.bk = lds + 2u * (l.k4 + l.pc + kDummySlots);
  l.bi = l.bk + l.k4;
  l.hist = l.bi + l.k4;
  l.ordt = l.hist + 2u * kBins;
  return l;
}

// The entries of one compaction: survivors (n0, possibly none) and appended entries (n1),
// each visited in groups of four (the slots up to a multiple of four exist; padding is skipped).
struct Segs {
  uint32_t *k0, *i0, *k1, *i1;
  uint32_t n0, n1;
};

__device__ __forceinline__ Segs make_segs(uint32_t* k0, uint32_t* i0, uint32_t n0, uint32_t* k1, uint32_t* i1,
                                          uint32_t n1) {
  Segs s;
  s.k0 = k0;
  s.i0 = i0;
  s.k1 = k1;
  s.i1 = i1;
  s.n0 = n0;
  s.n1 = n1;
  return s;
}

// Word of histogram bin b: bits 2-4 of the index are xored with bits 5-7. Neighbouring bins
// stay in neighbouring words (the counting atomics), and the 16-byte reads of the bin scan
// (lane l reads the four-bin groups of bins [32*(63-l), 32*(64-l))) hit eight different bank
// groups instead of one.
__device__ __forceinline__ uint32_t hslot(uint32_t b) { return b ^ (((b >> 5) & 7u) << 2); }

// One wave finds the bin of a kBins histogram (higher bin = better entries) that holds the
// `need`-th best entry: `above` entries lie in higher bins and `cnt` in that bin. Lane l sums
// the 32 bins of block 63 - l in groups of four; a wave scan finds the lane, the lane's group
// sums find the group, and one broadcast read finds the bin. Counting the prefix sums below
// `need` replaces searching, so the wave never diverges.
__device__ __forceinline__ void scan_select(const uint32_t* h, uint32_t need, uint32_t lane, uint32_t& bin,
                                            uint32_t& above, uint32_t& cnt) {
  constexpr uint32_t Q = kPer / 4;
  const uint32_t hb = 63u - lane, sw = hb & 7u;
  uint32_t gs[Q];  // gs[0]: the lane's highest four bins
  uint32_t s = 0;
#pragma unroll
  for (uint32_t j = 0; j < Q; ++j) {
    const uint4 q = *reinterpret_cast<const uint4*>(h + 32u * hb + 4u * ((Q - 1u - j) ^ sw));
    gs[j] = q.x + q.y + q.z + q.w;
    s += gs[j];
  }
  const uint32_t incl = wave_incl_scan(s);
  const uint64_t ge = ballot(incl >= need);
  const uint32_t src = ge ? static_cast<uint32_t>(__builtin_ctzll(ge)) : 63u;
  uint32_t acc = incl - s, gj = 0, gacc = incl - s;
#pragma unroll
  for (uint32_t j = 0; j < Q; ++j) {  // groups whose running total stays below need are passed
    acc += gs[j];
    const bool below = acc < need;
    gj += below ? 1u : 0u;
    gacc = below ? acc : gacc;
  }
  gj = __builtin_amdgcn_readlane(gj, src);
  gacc = __builtin_amdgcn_readlane(gacc, src);
  gj = gj < Q ? gj : Q - 1u;
  const uint32_t hs = 63u - src;
  const uint4 q = *reinterpret_cast<const uint4*>(h + 32u * hs + 4u * ((Q - 1u - gj) ^ (hs & 7u)));
  const uint32_t c[4] = {q.w, q.z, q.y, q.x};  // the group's bins, highest first
  uint32_t a = gacc, bi = 0, ab = gacc;
#pragma unroll
  for (uint32_t i = 0; i < 3; ++i) {
    a += c[i];
    const bool below = a < need;
    bi += below ? 1u : 0u;
    ab = below ? a : ab;
  }
  bin = 32u * hs + 4u * (Q - 1u - gj) + 3u - bi;
  above = ab;
  cnt = bi == 0 ? c[0] : bi == 1 ? c[1] : bi == 2 ? c[2] : c[3];
}

// Radix-select compaction.
//
// Reduces the entries of `sg` to the k best under the composite order (key descending, then
// index ascending) and writes them, unordered, to (dk, di); when fewer than k entries exist
// all of them are written followed by sentinels (key 0, index ~0) up to round4(k). In-loop
// calls return the smallest survivor as the new threshold (tkey, tidx) and the largest key
// seen in maxkey.
//
// Search: the first pass is a kBins-bin histogram of value bins (vbin) over the window
// [value(vlo_key), value(vhi_key)] when vok and the window is usable; values above it count in
// the top bin. If the pivot's value bin holds more than kListCap entries, its exact key
// bounds are found by a search over keys and the search continues with key bins
// (min(key, hi) - lo) >> shift over a key window [lo, hi]; while the pivot bin holds more
// than kListCap entries the window shrinks to it and the histogram repeats; a bin that is a
// single key (ties) continues on the indices in [ilo, ihi] (smaller index = higher bin).
// Without value bins the first key window is [0, key_hi] or [T.key, previous maximum] with
// keys above the maximum counted in the top ("open") bin. Then the entries above the pivot
// are scattered to the destination, the pivot bin's entries are gathered in a short list, and
// the list is ranked to place the rest and find the threshold.
//
// With so (final call only) and a single value pass, the survivors are written sorted to
// *so instead (sorted = true): a counting sort over the value bins (see below). A final call
// with at most kFinalPer entries per thread takes the one-pass form of it (final_sorted),
// which may use cbuf (room for round4(k) + 4 composites and k words after them: the append
// buffer, whose two arrays hold 2 (round4(k) + B + B2) words at least, with B + B2 >= k)
// and falls back to the above when a bin is too full.
//
// Barriers: two per histogram pass (after the counts; after the scan result is published),
// one after the scatter and one after the list is ranked.

// Adds one group's four counts (cnt[q] in {0, 1}) to their bins (bin[q]), one atomic per
// run of equal neighbouring bins: entries next to each other in the buffer are usually
// neighbours in the stream, and on rows with long runs of equal values this turns thousands
// of same-address atomics into a few.
__device__ __forceinline__ void add_runs(uint32_t* h, const uint32_t (&bin)[4], const uint32_t (&cnt)[4]) {
  uint32_t emit[4];
  uint32_t acc = cnt[3];
#pragma unroll
  for (int q = 2; q >= 0; --q) {
    const bool same = bin[q] == bin[q + 1];
    emit[q + 1] = same ? 0u : acc;
    acc = same ? acc + cnt[q] : cnt[q];
  }
  emit[0] = acc;
#pragma unroll
  for (uint32_t q = 0; q < 4; ++q)
    if (emit[q]) atomicAdd(&h[hslot(bin[q])], emit[q]);
}

// Group g of the compaction's entries: the appended segment's groups come first, then the
// survivors'. Sets the group's key and index pointers and returns how many of its four
// slots hold entries (the slots up to a multiple of four exist).
__device__ __forceinline__ uint32_t group_at(const Segs& sg, uint32_t g, uint32_t g1, uint32_t*& kp, uint32_t*& ip) {
  const bool app = g < g1;
  const uint32_t h = app ? g : g - g1;
  kp = (app ? sg.k1 : sg.k0) + 4u * h;
  ip = (app ? sg.i1 : sg.i0) + 4u * h;
  return min(4u, (app ? sg.n1 : sg.n0) - 4u * h);
}

// Histogram of all entries: value bins (vm), else key bins over the window; with raw, appended
// entries hold raw scores, which are replaced by their keys on the way. Returns this thread's
// largest key. Two groups per step, so both reads are in flight together.
template <int DT>
__device__ __forceinline__ uint32_t hist_all(const Segs& sg, uint32_t tid, uint32_t nt, uint32_t plo, uint32_t phi,
                                             bool open, uint32_t shift, uint32_t* h, bool raw, bool vm,
                                             const VBins& vb) {
  const uint32_t g1 = (sg.n1 + 3u) / 4u, groups = g1 + (sg.n0 + 3u) / 4u;
  uint32_t mx = 0;
  for (uint32_t g = tid; g < groups; g += 2u * nt) {
    uint4 kk[2];
    uint32_t nv[2];
    uint32_t* kp[2];
#pragma unroll
    for (uint32_t u = 0; u < 2; ++u) {
      const uint32_t gu = g + u * nt;
      uint32_t* ip;
      nv[u] = 0;
      kk[u] = make_uint4(0, 0, 0, 0);
      if (gu < groups) {
        nv[u] = group_at(sg, gu, g1, kp[u], ip);
        kk[u] = *reinterpret_cast<const uint4*>(kp[u]);
      }
    }
#pragma unroll
    for (uint32_t u = 0; u < 2; ++u) {
      if (raw && g + u * nt < g1) {
        kk[u] = make_uint4(key_of_score<DT>(kk[u].x), key_of_score<DT>(kk[u].y), key_of_score<DT>(kk[u].z),
                           key_of_score<DT>(kk[u].w));
        *lds_ptr(reinterpret_cast<u32x4*>(kp[u])) = u32x4{kk[u].x, kk[u].y, kk[u].z, kk[u].w};
      }
      if (vm) {
        // value bins spread entries: one atomic each, except where most lanes' groups fall
        // whole into one bin (a sorted stretch of the buffer, whose atomics would all hit a
        // few addresses): then each run of lanes with the same whole-group bin adds its
        // entries with one atomic, by the run's first lane
        uint32_t b[4];
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          const uint32_t key = u4get(kk[u], q);
          b[q] = vbin<DT>(key, vb);
          mx = q < nv[u] ? max(mx, key) : mx;
        }
        const bool same = nv[u] == 4u && b[0] == b[1] && b[1] == b[2] && b[2] == b[3];
        const uint32_t lane = tid & 63u;
        if (popc(ballot(same)) >= 16u) {
          const uint32_t rk = same ? b[0] : (0x80000000u | lane);  // a lane of its own otherwise
          const uint32_t prev = static_cast<uint32_t>(
              __builtin_amdgcn_ds_bpermute(static_cast<int>(((lane - 1u) & 63u) << 2), static_cast<int>(rk)));
          const bool first = lane == 0 || rk != prev;
          // runs end at the next run's first lane or at the first inactive lane
          const uint64_t stop = ballot(first) | ~ballot(true);
          if (same) {
            if (first) {
              const uint64_t rest = lane == 63u ? 0ull : stop >> (lane + 1u);
              const uint32_t len = rest ? static_cast<uint32_t>(__builtin_ctzll(rest)) + 1u : 64u - lane;
              atomicAdd(&h[hslot(b[0])], 4u * len);
            }
          } else {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q)
              if (q < nv[u]) atomicAdd(&h[hslot(b[q])], 1u);
          }
        } else {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q)
            if (q < nv[u]) atomicAdd(&h[hslot(b[q])], 1u);
        }
      } else {  // key bins: runs of equal keys are common (ties), one atomic per run
        uint32_t bin[4], cnt[4];
#pragma unroll
        for (uint32_t q = 0; q < 4; ++q) {
          const uint32_t key = u4get(kk[u], q);
          const bool valid = q < nv[u];
          mx = valid ? max(mx, key) : mx;
          bin[q] = (min(key, phi) - plo) >> shift;
          cnt[q] = (valid && key >= plo && (key <= phi || open)) ? 1u : 0u;
        }
        add_runs(h, bin, cnt);
      }
    }
  }
  return mx;
}

// Histogram of the indices of the entries whose key is pkey.
__device__ __forceinline__ void ties_all(const Segs& sg, uint32_t tid, uint32_t nt, uint32_t pkey, uint32_t iplo,
                                         uint32_t iphi, uint32_t shift, uint32_t* h) {
  const uint32_t g1 = (sg.n1 + 3u) / 4u, groups = g1 + (sg.n0 + 3u) / 4u;
  for (uint32_t g = tid; g < groups; g += nt) {
    uint32_t *kp, *ip;
    const uint32_t nv = group_at(sg, g, g1, kp, ip);
    const uint4 kk = *reinterpret_cast<const uint4*>(kp);
    const uint4 ii = *reinterpret_cast<const uint4*>(ip);
    uint32_t bin[4], cnt[4];
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
      const uint32_t key = u4get(kk, q), id = u4get(ii, q);
      bin[q] = kBins - 1u - ((id - iplo) >> shift);
      cnt[q] = (q < nv && key == pkey && id >= iplo && id <= iphi) ? 1u : 0u;
    }
    add_runs(h, bin, cnt);
  }
}

// Stores entry c (a composite) at position `at` of the outputs, or, with pairs, as a (key,
// index) pair at pairs[at].
template <int DT>
__device__ __forceinline__ void store_out(void* out_vals, IdxOut out_idx, uint2* pairs, uint64_t at, uint64_t c) {
  const uint32_t key = static_cast<uint32_t>(c >> 32), id = ~static_cast<uint32_t>(c);
  if (pairs) {
    pairs[at] = make_uint2(key, id);
    return;
  }
  if (out_vals) {
    if constexpr (DT == DS_BF16)
      static_cast<uint16_t*>(out_vals)[at] = static_cast<uint16_t>(raw_of_key<DT>(key));
    else
      static_cast<uint32_t*>(out_vals)[at] = raw_of_key<DT>(key);
  }
  if (out_idx.p) {
    if (out_idx.wide)  // sign-extended: padding (index ~0) reads -1 in either width
      static_cast<int64_t*>(out_idx.p)[at] = static_cast<int64_t>(static_cast<int32_t>(id));
    else
      static_cast<int32_t*>(out_idx.p)[at] = static_cast<int32_t>(id);
  }
}

// Where a final compaction may write its survivors directly, sorted: row `row` of the
// outputs, or pairs[row * k ...] when pairs is set.
struct OutSpec {
  void* vals;
  IdxOut idx;
  uint2* pairs;
  uint64_t row;
  bool on = true;  // false: the caller writes the survivors itself (no sorted output here)
};

// A final compaction sorts its survivors itself (a counting sort over its value bins) when
// no value bin above the pivot holds more entries than this.
constexpr uint32_t kSortedBinCap = 32;

// The pivot window a compaction ends with: value bin vbin_p (vm), else keys [plo, phi], or,
// for ties, key pkey with indices [iplo, iphi].
struct Pivot {
  uint32_t plo, phi, pkey, iplo, iphi, k, vbin_p;
  VBins vb;
  bool tie, vm;
};

// Scatter of all entries: those above the pivot window go to (dk, di), those inside it to
// the list.
// With bin_slots (value bins only), an entry above the pivot bin takes the next slot of its
// bin from bin_slots (each bin's first slot, highest bins first) instead of a slot in arrival
// order, so the destination ends up ordered by bin.
template <int DT>
__device__ __forceinline__ void scatter_all(const Segs& sg, uint32_t tid, uint32_t nt, uint32_t lane, const Pivot& pv,
                                            uint32_t* dk, uint32_t* di, Scalars& sc, uint32_t* bin_slots) {
  const uint32_t g1 = (sg.n1 + 3u) / 4u, groups = g1 + (sg.n0 + 3u) / 4u;
  const uint32_t iters = (groups + nt - 1u) / nt;
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t g = it * nt + tid;
    uint4 kk = make_uint4(0, 0, 0, 0), ii = make_uint4(0, 0, 0, 0);
    uint32_t nv = 0;
    if (g < groups) {
      uint32_t *kp, *ip;
      nv = group_at(sg, g, g1, kp, ip);
      kk = *reinterpret_cast<const uint4*>(kp);
      ii = *reinterpret_cast<const uint4*>(ip);
    }
    bool up[4], mid[4];
    uint64_t bu[4], bm[4];
    uint32_t nu = 0, nm = 0;
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
      const uint32_t key = u4get(kk, q), id = u4get(ii, q);
      const bool valid = q < nv;
      if (pv.vm) {
        const uint32_t b = vbin<DT>(key, pv.vb);
        up[q] = valid && b > pv.vbin_p;
        mid[q] = valid && b == pv.vbin_p;
        if (bin_slots && up[q]) {  // sorted mode: the bin's next slot
          const uint32_t at = __atomic_fetch_add(lds_ptr(&bin_slots[hslot(b)]), 1u, __ATOMIC_RELAXED);
          dk[at] = key;
          di[at] = id;
          up[q] = false;
        }
      } else if (!pv.tie) {
        up[q] = valid && key > pv.phi;
        mid[q] = valid && key >= pv.plo && key <= pv.phi;
      } else {
        up[q] = valid && (key > pv.pkey || (key == pv.pkey && id < pv.iplo));
        mid[q] = valid && key == pv.pkey && id >= pv.iplo && id <= pv.iphi;
      }
      bu[q] = ballot(up[q]);
      bm[q] = ballot(mid[q]);
      nu += popc(bu[q]);
      nm += popc(bm[q]);
    }
    if (nu | nm) {
      uint32_t b0 = 0, b1 = 0;
      if (lane == 0) {
        b0 = atomicAdd(&sc.outpos, nu);
        b1 = atomicAdd(&sc.listpos, nm);
      }
      b0 = uni(b0);
      b1 = uni(b1);
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) {
        if (up[q]) {
          const uint32_t at = mbcnt(bu[q], b0);
          if (at < pv.k) {
            dk[at] = u4get(kk, q);
            di[at] = u4get(ii, q);
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
}

// Entries per thread that the one-pass final sort keeps in registers.
constexpr uint32_t kFinalPer = 4;

// The value of a raw score (the bits of the element; for bf16 the element sits in the top
// half of the word): the same float as value_of_key(key_of_score(s)).
template <int DT>
__device__ __forceinline__ float value_of_score(uint32_t s) {
  if constexpr (DT == DS_BF16)
    return __uint_as_float(s & 0xFFFF0000u);
  else
    return __uint_as_float(s);
}

template <int DT>
__device__ __forceinline__ uint32_t vbin_of_value(float v, const VBins& vb) {
#pragma clang fp contract(off)
  const float t = (v - vb.lo) * vb.scale;
  return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(t, 0.0f, static_cast<float>(kBins - 1u)));
}

// One-pass final compaction with sorted output, for at most kFinalPer * NT entries and
// usable value bins (the common end of a stream). Every thread keeps up to kFinalPer
// entries in registers and takes each one's place in its value bin from the histogram's
// returning atomic (its arrival slot). All threads scan the bins together (BPT bins each,
// then the wave totals); the bin that holds the k-th best entry is the pivot bin, and each
// bin above it gets its first output slot (higher bins first). An entry above the pivot bin
// is stored as a composite at its bin's first slot plus its arrival slot in cbuf, then ranked
// against its bin's entries for its output position; the pivot bin's entries (a short list)
// are ranked by one wave. When the pivot bin holds more than kListCap entries or a bin above
// it more than kSortedBinCap, false is returned before any output is written, and the pass is
// handed to the general compaction as its first value pass (the histogram in its layout, the
// appended entries converted to keys in place, the waves' largest keys in sc.red). The
// histograms here are plain (bin b at index b) until then; on success both are left dirty
// (this is a stream's last compaction).
// h is the current histogram (zero on entry), hs the other one; cbuf has room for k + 3
// composites and then k bin numbers (cbin, from slot round4(k) + 4 of cbuf) and may overlap the
// entries (they are all in registers before it is written).
template <int WAVES, int DT, bool RAW>
__device__ __forceinline__ bool final_sorted(const Segs& sg, uint32_t k, const OutSpec so, const VBins& vb,
                                             uint32_t* h, uint32_t* hs, uint64_t* cbuf, Scalars& sc,
                                             uint32_t& tkey, uint32_t& tidx) {
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t BPT = kBins / NT;  // bins per thread in the scan
  static_assert(kBins % NT == 0 && BPT >= 2 && BPT <= 32, "bins per thread");
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t n = sg.n0 + sg.n1;  // k < n <= kFinalPer * NT

  // histogram with arrival slots; the entries stay in registers
  uint32_t key[kFinalPer], id[kFinalPer], bin[kFinalPer], arr[kFinalPer];
#pragma unroll
  for (uint32_t j = 0; j < kFinalPer; ++j) {
    const uint32_t e = tid + j * NT;
    key[j] = 0;
    id[j] = kSentinelIdx;
    bin[j] = 0;
    arr[j] = 0;
    if (j * NT < n && e < n) {
      const bool app = e < sg.n1;
      const uint32_t w = app ? sg.k1[e] : sg.k0[e - sg.n1];
      id[j] = app ? sg.i1[e] : sg.i0[e - sg.n1];
      const bool raw = RAW && app;
      key[j] = raw ? key_of_score<DT>(w) : w;
      bin[j] = vbin_of_value<DT>(raw ? value_of_score<DT>(w) : value_of_key<DT>(w), vb);
      arr[j] = __atomic_fetch_add(lds_ptr(&h[bin[j]]), 1u, __ATOMIC_RELAXED);
    }
  }
  if (tid == 0) sc.big = 0;
  lds_sync();

  // bin scan: thread t holds bins [kBins - BPT (t + 1), kBins - BPT t), highest first in c[]
  const uint32_t lo = kBins - BPT * (tid + 1u);
  uint32_t c[BPT];
#pragma unroll
  for (uint32_t g = 0; g < BPT / 2; ++g) {
    const uint2 q = *reinterpret_cast<const uint2*>(h + lo + 2u * g);
    c[BPT - 1u - 2u * g] = q.x;
    c[BPT - 2u - 2u * g] = q.y;
  }
  uint32_t s = 0;
#pragma unroll
  for (uint32_t i = 0; i < BPT; ++i) s += c[i];
  const uint32_t incl = wave_incl_scan(s);
  if (lane == 63) sc.red[wave] = incl;
  lds_sync();
  // entries in higher bins: this wave's lanes below, then the earlier waves (an inclusive
  // scan of the wave totals over the first lanes, read at the previous wave)
  uint32_t wt = lane < static_cast<uint32_t>(WAVES) ? sc.red[lane] : 0u;
  wt += __builtin_amdgcn_update_dpp(0u, wt, 0x111, 0xF, 0xF, true);
  wt += __builtin_amdgcn_update_dpp(0u, wt, 0x112, 0xF, 0xF, true);
  wt += __builtin_amdgcn_update_dpp(0u, wt, 0x114, 0xF, 0xF, true);
  wt += __builtin_amdgcn_update_dpp(0u, wt, 0x118, 0xF, 0xF, true);
  static_assert(WAVES <= 16, "wave totals scanned within one row of lanes");
  const uint32_t wv = uni(wave);
  uint32_t start = incl - s + (wv ? __builtin_amdgcn_readlane(wt, wv - 1u) : 0u);
  uint32_t st[BPT];
  bool big = false;
#pragma unroll
  for (uint32_t i = 0; i < BPT; ++i) {
    st[i] = start;
    const uint32_t end = start + c[i];
    if (start < k && end >= k) {  // the pivot bin: it holds rank k - 1 (ranks from 0, best first)
      sc.pub[0] = lo + BPT - 1u - i;
      sc.pub[1] = start;
      sc.pub[2] = c[i];
      big = big || c[i] > kListCap;
    } else if (end < k) {
      big = big || c[i] > kSortedBinCap;
    }
    start = end;
  }
#pragma unroll
  for (uint32_t g = 0; g < BPT / 2; ++g)
    *reinterpret_cast<uint2*>(hs + lo + 2u * g) = make_uint2(st[BPT - 1u - 2u * g], st[BPT - 2u - 2u * g]);
  if (big) sc.big = 1;
  lds_sync();
  if (sc.big) {
    // Hand this pass to the general compaction as its first value pass: the counts in its
    // bin layout (every read of h was before the last barrier but one), the other histogram
    // zero, the appended entries as keys, and each wave's largest key.
#pragma unroll
    for (uint32_t i = 0; i < BPT; ++i) {
      h[hslot(lo + BPT - 1u - i)] = c[i];
      hs[lo + i] = 0;
    }
    uint32_t mx = 0;
#pragma unroll
    for (uint32_t j = 0; j < kFinalPer; ++j) {
      const uint32_t e = tid + j * NT;
      if (j * NT < n && e < n) {
        mx = max(mx, key[j]);
        if (RAW && e < sg.n1) sg.k1[e] = key[j];
      }
    }
    mx = wave_max32(mx);
    if (lane == 0) sc.red[wave] = mx;
    lds_sync();
    return false;
  }
  const uint32_t pbin = sc.pub[0], above = sc.pub[1], pcnt = sc.pub[2];

  // entries above the pivot bin to their bins' slots (with their bins, in cbin), the pivot
  // bin's to the list
  uint32_t* const cbin = reinterpret_cast<uint32_t*>(cbuf + round4(k) + 4u);
#pragma unroll
  for (uint32_t j = 0; j < kFinalPer; ++j) {
    if (j * NT < n && tid + j * NT < n) {
      if (bin[j] > pbin) {
        const uint32_t d = hs[bin[j]] + arr[j];
        cbuf[d] = comp_of(key[j], id[j]);
        cbin[d] = bin[j];
      } else if (bin[j] == pbin) {
        sc.lkey[arr[j]] = key[j];
        sc.lidx[arr[j]] = id[j];
      }
    }
  }
  lds_sync();

  // the entry at slot p: its bin's first slot plus the bin's entries that rank above it. Slots
  // go in order to the threads from wave 1 on, so a wave's lanes share a few neighbouring bins
  // and only the waves that hold the crowded bins loop long; wave 0 ranks the pivot bin's list
  for (uint32_t p = tid - 64u; tid >= 64u && p < above; p += NT - 64u) {
    const uint64_t me = cbuf[p];
    const uint32_t b = cbin[p];
    const uint32_t s0 = hs[b], end = s0 + h[b];
    uint32_t r = 0;
    for (uint32_t m = s0; m < end; m += 4u) {
      // four at a time: the reads past the bin's end (masked out) stay inside cbuf's k + 3
      // slots, since the bin ends at most at slot k - 1
      uint64_t o[4];
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) o[u] = cbuf[m + u];
#pragma unroll
      for (uint32_t u = 0; u < 4; ++u) r += (m + u < end && o[u] > me) ? 1u : 0u;
    }
    store_out<DT>(so.vals, so.idx, so.pairs, so.row * k + s0 + r, me);
  }
  // the pivot bin's list: the k - above best of it follow the entries above it (wave 0, the
  // oldest of its SIMD, which the SIMD serves first)
  if (wave == 0) {
    const bool have = lane < pcnt;
    const uint32_t lk = have ? sc.lkey[lane] : 0u, li = have ? sc.lidx[lane] : kSentinelIdx;
    const uint64_t mine = comp_of(lk, li);
    uint32_t rank = 0;
    for (uint32_t m = 0; m < pcnt; ++m) rank += readlane64(mine, m) > mine ? 1u : 0u;
    const uint32_t need = k - above;
    if (have && rank < need) store_out<DT>(so.vals, so.idx, so.pairs, so.row * k + above + rank, mine);
    const uint64_t piv = ballot(have && rank == need - 1u);
    const uint32_t pl = piv ? static_cast<uint32_t>(__builtin_ctzll(piv)) : 0u;
    if (lane == 0) {
      sc.pub[3] = __builtin_amdgcn_readlane(lk, pl);
      sc.pub[4] = __builtin_amdgcn_readlane(li, pl);
      ++sc.st_p;
    }
  }
  lds_sync();
  tkey = sc.pub[3];
  tidx = sc.pub[4];
  return true;
}

template <int WAVES, int DT, bool RAW>
__device__ void compact(const Segs& sg, uint32_t* dk, uint32_t* di, uint32_t k, bool fin, bool have_t,
                        uint32_t key_hi, uint32_t ilo, uint32_t ihi, Scalars& sc, uint32_t* hist2, uint32_t& hpar,
                        uint32_t& tkey, uint32_t& tidx, uint32_t& maxkey, uint32_t vlo_key, uint32_t vhi_key,
                        bool vok, const OutSpec* so, bool& sorted, uint32_t* clear, uint64_t* cbuf) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t n = sg.n0 + sg.n1;

  sorted = false;
  if (n <= k) {  // keep everything (only the final call can get here)
    const uint32_t k4 = round4(k);
    for (uint32_t i = tid; i < k4; i += NT) {
      uint32_t key = 0, id = kSentinelIdx;
      if (i < sg.n0) {
        key = sg.k0[i];
        id = sg.i0[i];
      } else if (i < n) {
        key = sg.k1[i - sg.n0];
        if (RAW) key = key_of_score<DT>(key);
        id = sg.i1[i - sg.n0];
      }
      dk[i] = key;
      di[i] = id;
    }
    lds_sync();
    return;
  }
  if (tid == 0) {  // last used by the previous compaction's scatter, several barriers ago
    sc.outpos = 0;
    sc.listpos = 0;
  }

  Pivot pv;
  pv.plo = have_t ? tkey : 0u;
  pv.phi = have_t ? maxkey : key_hi;
  pv.tie = false;
  pv.pkey = 0;
  pv.iplo = ilo;
  pv.iphi = ihi;
  pv.k = k;
  pv.vbin_p = 0;
  pv.vm = vok && vbins_of<DT>(vlo_key, vhi_key, pv.vb);
  bool one_pass = fin && so && so->on && pv.vm && n <= kFinalPer * NT;
  if (one_pass &&
      final_sorted<WAVES, DT, RAW>(sg, k, *so, pv.vb, hist2 + kBins * (hpar & 1u), hist2 + kBins * ((hpar + 1u) & 1u),
                                   cbuf, sc, tkey, tidx)) {
    sorted = true;
    return;
  }
  bool open = have_t, first = true;
  uint32_t need = k, above_total = 0, cnt = 0, seen_max = 0;
  for (;;) {
    const uint32_t bl = bitlen32(pv.tie ? pv.iphi - pv.iplo : pv.phi - pv.plo);
    const uint32_t shift = bl > kLogBins ? bl - kLogBins : 0u;
    uint32_t* h = hist2 + kBins * (hpar & 1u);
    uint32_t* hz = hist2 + kBins * ((hpar + 1u) & 1u);
    if (!one_pass) {  // else the one-pass form already made this (first) pass
      // the other histogram was last read by the previous scan, before the last barrier
      for (uint32_t b = 4u * tid; b < kBins; b += 4u * NT) *reinterpret_cast<uint4*>(hz + b) = make_uint4(0, 0, 0, 0);
      if (!pv.tie) {
        uint32_t mx = hist_all<DT>(sg, tid, NT, pv.plo, pv.phi, open, shift, h, RAW && first, pv.vm, pv.vb);
        if (first) {
          mx = wave_max32(mx);
          if (lane == 0) sc.red[wave] = mx;
        }
      } else {
        ties_all(sg, tid, NT, pv.pkey, pv.iplo, pv.iphi, shift, h);
      }
      lds_sync();
    }
    one_pass = false;
    ++hpar;
    if (tid == 0) ++sc.st_p;
    if (wave == 0) {
      uint32_t smax = 0;
      if (first) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) smax = max(smax, sc.red[w]);
      }
      uint32_t bin, above, c;
      scan_select(h, need, lane, bin, above, c);
      uint32_t blo = 0, bhi = 0;
      if (so && so->on && fin && pv.vm && c <= kListCap) {
        // Counting sort for the output: each bin above the pivot gets its first slot (the
        // entries of the higher bins come first), written over its count, and blo becomes
        // the largest such count. Lane l holds bins [32 (63 - l), 32 (64 - l)).
        // (16-byte groups of four bins at the bin scan's swizzled addresses; in a group the
        // lowest bin comes first)
        constexpr uint32_t Q = kPer / 4;
        const uint32_t hb = 63u - lane, sw = hb & 7u;
        uint4 g[Q];  // g[0]: the lane's highest four bins
        uint32_t lsum = 0, lmax = 0;
#pragma unroll
        for (uint32_t j = 0; j < Q; ++j) {
          g[j] = *reinterpret_cast<const uint4*>(h + 32u * hb + 4u * ((Q - 1u - j) ^ sw));
          const uint32_t b0 = 32u * hb + 4u * (Q - 1u - j);
          lsum += g[j].x + g[j].y + g[j].z + g[j].w;
          lmax = b0 + 3u > bin ? max(lmax, g[j].w) : lmax;
          lmax = b0 + 2u > bin ? max(lmax, g[j].z) : lmax;
          lmax = b0 + 1u > bin ? max(lmax, g[j].y) : lmax;
          lmax = b0 > bin ? max(lmax, g[j].x) : lmax;
        }
        uint32_t off = wave_incl_scan(lsum) - lsum;
#pragma unroll
        for (uint32_t j = 0; j < Q; ++j) {
          uint4 o;
          o.w = off;
          off += g[j].w;
          o.z = off;
          off += g[j].z;
          o.y = off;
          off += g[j].y;
          o.x = off;
          off += g[j].x;
          *reinterpret_cast<uint4*>(h + 32u * hb + 4u * ((Q - 1u - j) ^ sw)) = o;
        }
        blo = wave_max32(lmax);
      }
      if (pv.vm && c > kListCap) {  // the key range of the value bin, for the key passes
        blo = static_cast<uint32_t>(vbin_first_key<DT>(bin, vlo_key, key_of_inf<DT>(), pv.vb, lane));
        bhi = bin + 1u < kBins
                  ? static_cast<uint32_t>(vbin_first_key<DT>(bin + 1u, vlo_key, key_of_inf<DT>(), pv.vb, lane) - 1u)
                  : key_of_inf<DT>();
      }
      if (lane == 0) {
        sc.pub[0] = bin;
        sc.pub[1] = above;
        sc.pub[2] = c;
        sc.pub[3] = smax;
        sc.pub[4] = blo;
        sc.pub[5] = bhi;
      }
    }
    lds_sync();
    const uint32_t bin = sc.pub[0], above = sc.pub[1];
    cnt = sc.pub[2];
    if (first) seen_max = sc.pub[3];
    first = false;
    need -= above;
    above_total += above;
    if (pv.vm) {
      if (cnt <= kListCap) {
        pv.vbin_p = bin;
        break;
      }
      // continue with key bins over the value bin's keys (all of them <= the largest key)
      pv.vm = false;
      open = false;
      pv.plo = sc.pub[4];
      pv.phi = min(sc.pub[5], seen_max);
      if (pv.plo == pv.phi) {
        pv.tie = true;
        pv.pkey = pv.plo;
      }
    } else if (!pv.tie) {
      const bool open_bin = open && bin == ((pv.phi - pv.plo) >> shift);
      const uint32_t nlo = pv.plo + (bin << shift);
      const uint64_t nhi64 = static_cast<uint64_t>(nlo) + (1ull << shift) - 1u;
      pv.phi = open_bin ? seen_max : (nhi64 > pv.phi ? pv.phi : static_cast<uint32_t>(nhi64));
      pv.plo = nlo;
      open = false;
      if (cnt <= kListCap) break;
      if (pv.plo == pv.phi) {  // one key holds more than kListCap entries: continue on indices
        pv.tie = true;
        pv.pkey = pv.plo;
      }
    } else {
      const uint32_t nlo = pv.iplo + ((kBins - 1u - bin) << shift);
      const uint64_t nhi64 = static_cast<uint64_t>(nlo) + (1ull << shift) - 1u;
      pv.iphi = nhi64 > pv.iphi ? pv.iphi : static_cast<uint32_t>(nhi64);
      pv.iplo = nlo;
      if (cnt <= kListCap || shift == 0) break;
    }
  }
  cnt = cnt < kListCap ? cnt : kListCap;  // more only if (key, index) pairs repeat
  // the final pass's histogram holds bin slots when the output can be sorted here
  uint32_t* const slots = hist2 + kBins * ((hpar + 1u) & 1u);
  const bool srt = so && so->on && fin && pv.vm && sc.pub[4] <= kSortedBinCap;

  // scatter: entries above the pivot window go to the destination, the window's to the list
  scatter_all<DT>(sg, tid, NT, lane, pv, dk, di, sc, srt ? slots : nullptr);
  lds_sync();

  // wave 0 ranks the short list, places the `need` best of it after the above_total entries
  // and publishes the threshold
  if (wave == 0) {
    const bool have = lane < cnt;
    const uint32_t lk = have ? sc.lkey[lane] : 0u, li = have ? sc.lidx[lane] : kSentinelIdx;
    const uint64_t mine = comp_of(lk, li);
    uint32_t rank = 0;
    for (uint32_t m = 0; m < cnt; ++m) rank += readlane64(mine, m) > mine ? 1u : 0u;
    if (have && rank < need) {
      if (srt) {
        store_out<DT>(so->vals, so->idx, so->pairs, so->row * k + above_total + rank, mine);
      } else {
        dk[above_total + rank] = lk;
        di[above_total + rank] = li;
      }
    }
    const uint64_t piv = ballot(have && rank == need - 1u);
    const uint32_t pl = piv ? static_cast<uint32_t>(__builtin_ctzll(piv)) : 0u;
    if (lane == 0) {
      sc.pub[0] = __builtin_amdgcn_readlane(lk, pl);
      sc.pub[1] = __builtin_amdgcn_readlane(li, pl);
    }
  }
  if (srt) {
    // each entry above the pivot bin sits inside its bin's slots, [end of the next higher
    // bin, end of its bin); its place is the bin's start plus the entries of the bin that
    // rank above it
    for (uint32_t s = tid; s < above_total; s += NT) {
      const uint32_t key = dk[s], id = di[s];
      const uint32_t b = vbin<DT>(key, pv.vb);
      const uint32_t end = slots[hslot(b)], start = b + 1u < kBins ? slots[hslot(b + 1u)] : 0u;
      const uint64_t c = comp_of(key, id);
      uint32_t r = 0;
      for (uint32_t j = start; j < end; ++j) r += comp_of(dk[j], di[j]) > c ? 1u : 0u;
      store_out<DT>(so->vals, so->idx, so->pairs, so->row * k + start + r, c);
    }
    sorted = true;
  }
  if (clear && tid == 0) *clear = 0;  // before the last barrier: no wave appends before it
  lds_sync();
  tkey = sc.pub[0];
  tidx = sc.pub[1];
  maxkey = seen_max;
}

// --------------------------------------------------------------------------- final sort
// Compare-exchange stages (SIZE, STRIDE) of a bitonic sort, best first, of TOTAL 64-bit keys
// held E per thread in registers (element t*E + j in thread t). Partners closer than E are
// in the same thread, closer than 64*E in the same wave (lane exchanges); farther partners
// go through LDS (xk / xi take the high / low halves) between two barriers. Recurses
// through all later stages.
template <int E, uint32_t TOTAL, uint32_t SIZE, uint32_t STRIDE>
__device__ __forceinline__ void bitonic(uint64_t (&v)[E], uint32_t* xk, uint32_t* xi, uint32_t t, uint32_t lane) {
  if constexpr (STRIDE < static_cast<uint32_t>(E)) {
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      if ((j & STRIDE) == 0) {
        const bool desc = ((t * E + j) & SIZE) == 0;
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
      const uint32_t e = t * E + j;
      const bool take_max = ((e & STRIDE) == 0) == ((e & SIZE) == 0);
      const uint64_t o = xor_lane64(v[j], M, lane);
      v[j] = take_max ? (o > v[j] ? o : v[j]) : (o < v[j] ? o : v[j]);
    }
  } else {
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      xk[t * E + j] = static_cast<uint32_t>(v[j] >> 32);
      xi[t * E + j] = static_cast<uint32_t>(v[j]);
    }
    lds_sync();
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      const uint32_t e = t * E + j;
      const bool take_max = ((e & STRIDE) == 0) == ((e & SIZE) == 0);
      const uint64_t o = (static_cast<uint64_t>(xk[e ^ STRIDE]) << 32) | xi[e ^ STRIDE];
      v[j] = take_max ? (o > v[j] ? o : v[j]) : (o < v[j] ? o : v[j]);
    }
    lds_sync();
  }
  if constexpr (STRIDE > 1)
    bitonic<E, TOTAL, SIZE, STRIDE / 2>(v, xk, xi, t, lane);
  else if constexpr (SIZE < TOTAL)
    bitonic<E, TOTAL, SIZE * 2, SIZE>(v, xk, xi, t, lane);
}

// Number of barriers the network above executes.
template <int E, uint32_t TOTAL>
constexpr int bitonic_barriers() {
  int c = 0;
  for (uint32_t size = 2; size <= TOTAL; size <<= 1)
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1)
      if (stride >= 64u * E) c += 2;
  return c;
}

// Sorts the k entries (fk, fi) (k <= 2^LOGT, padded with zeros) best first and stores them.
// TH = min(2^LOGT, workgroup) threads hold E = 2^LOGT / TH entries each; the other waves only
// take part in the barriers. (xk, xi) must not overlap
// (fk, fi) and hold 2^LOGT words each.
template <int DT, int WAVES, uint32_t LOGT>
__device__ __forceinline__ void sort_store_t(const uint32_t* fk, const uint32_t* fi, uint32_t* xk, uint32_t* xi, uint32_t k,
                             void* out_vals, IdxOut out_idx, uint2* pairs, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64, TOTAL = 1u << LOGT;
  constexpr uint32_t TH = TOTAL > NT ? NT : TOTAL;
  constexpr int E = static_cast<int>(TOTAL / TH);
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  if (tid < TH) {
    uint64_t v[E];
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      const uint32_t e = tid * E + j;
      v[j] = e < k ? comp_of(fk[e], fi[e]) : 0ull;
    }
    bitonic<E, TOTAL, 2, 1>(v, xk, xi, tid, lane);
#pragma unroll
    for (uint32_t j = 0; j < static_cast<uint32_t>(E); ++j) {
      const uint32_t e = tid * E + j;
      if (e < k) store_out<DT>(out_vals, out_idx, pairs, row * k + e, v[j]);
    }
  } else {
    constexpr int NB = bitonic_barriers<E, TOTAL>();
    for (int s = 0; s < NB; ++s) lds_sync();
  }
}

// Bitonic sort in LDS with one barrier per stage, for large k in small workgroups: sorts cap
// (a power of two >= k) composites held as (xk, xi) halves, best first, and stores the first k.
template <int DT, int WAVES>
__device__ __forceinline__ void sort_store_lds(const uint32_t* fk, const uint32_t* fi, uint32_t* xk, uint32_t* xi, uint32_t k,
                               uint32_t cap, void* out_vals, IdxOut out_idx, uint2* pairs, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < cap; i += NT) {
    xk[i] = i < k ? fk[i] : 0u;
    xi[i] = i < k ? ~fi[i] : 0u;
  }
  lds_sync();
  for (uint32_t size = 2; size <= cap; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t q = tid; q < cap / 2; q += NT) {
        const uint32_t i = ((q & ~(stride - 1)) << 1) | (q & (stride - 1));
        const uint32_t j = i + stride;
        const uint64_t a = (static_cast<uint64_t>(xk[i]) << 32) | xi[i];
        const uint64_t b = (static_cast<uint64_t>(xk[j]) << 32) | xi[j];
        const bool desc = (i & size) == 0;
        if (desc ? b > a : a > b) {
          xk[i] = static_cast<uint32_t>(b >> 32);
          xi[i] = static_cast<uint32_t>(b);
          xk[j] = static_cast<uint32_t>(a >> 32);
          xi[j] = static_cast<uint32_t>(a);
        }
      }
      lds_sync();
    }
  }
  for (uint32_t i = tid; i < k; i += NT)
    store_out<DT>(out_vals, out_idx, pairs, row * k + i, (static_cast<uint64_t>(xk[i]) << 32) | xi[i]);
}

// Sort by runs and pairwise merges, for k <= 64 * kMaxRuns: every wave sorts runs of 64
// entries in registers (a bitonic network over lane exchanges, best first), then RUNS runs
// (a power of two; runs past k hold zero padding, which ranks below every element) are
// merged in pairs until one is left. In a merge an entry's place is its position in its run
// plus the number of entries of the partner run that rank above it (a binary search; equal
// entries of the earlier run count as above, so equal padding gets distinct places). Each
// round reads one half of xs and writes the other (xs: 2 * 64 * RUNS 64-bit words); the last
// round stores the places below k.
constexpr uint32_t kMaxRuns = 16;

// Bitonic sort of one value per lane over the 64 lanes, largest first.
__device__ __forceinline__ uint64_t wave_sort64(uint64_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = xor_lane64(v, stride, lane);
      const bool take_max = ((lane & stride) == 0) == ((lane & size) == 0);
      v = ((o > v) == take_max) ? o : v;
    }
  }
  return v;
}

template <int DT, int WAVES, uint32_t RUNS>
__device__ __forceinline__ void sort_runs_store(const uint32_t* fk, const uint32_t* fi, uint64_t* xs, uint32_t k,
                                                void* out_vals, IdxOut out_idx, uint2* pairs, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64, N = 64 * RUNS;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  if constexpr (RUNS == 1) {
    if (wave == 0) {
      const uint64_t v = wave_sort64(lane < k ? comp_of(fk[lane], fi[lane]) : 0ull, lane);
      if (lane < k) store_out<DT>(out_vals, out_idx, pairs, row * k + lane, v);
    }
    return;
  }
  __attribute__((address_space(3))) uint64_t* src = lds_ptr(xs);
  __attribute__((address_space(3))) uint64_t* dst = src + N;
  for (uint32_t r = wave; r < RUNS; r += WAVES) {
    const uint32_t e = 64u * r + lane;
    src[e] = wave_sort64(e < k ? comp_of(fk[e], fi[e]) : 0ull, lane);
  }
  lds_sync();
#pragma unroll
  for (uint32_t L = 64; L < N; L <<= 1) {
    const bool last = 2u * L == N;
    for (uint32_t e = tid; e < N; e += NT) {
      const uint32_t r = e / L, i = e % L, pb = (r ^ 1u) * L;
      const bool before = (r & 1u) != 0;  // the partner run comes first
      const uint64_t c = src[e];
      uint32_t pos = 0;
#pragma unroll
      for (uint32_t step = L; step > 0; step >>= 1) {
        const uint64_t x = src[pb + min(pos + step, L) - 1u];
        const bool above = x > c || (before && x == c);
        pos = (pos + step <= L && above) ? pos + step : pos;
      }
      const uint32_t at = (r & ~1u) * L + i + pos;
      if (last) {
        if (at < k) store_out<DT>(out_vals, out_idx, pairs, row * k + at, c);
      } else {
        dst[at] = c;
      }
    }
    if (!last) {
      lds_sync();
      __attribute__((address_space(3))) uint64_t* t = src;
      src = dst;
      dst = t;
    }
  }
}

// Sort of the k final entries, best first: by runs and ranks up to 64 * kMaxRuns entries
// (xs: 64-bit scratch), the register bitonic sort when at most eight entries per thread are
// needed, else the LDS bitonic sort. The sorted entries go to row `row` of the outputs, or,
// with pairs, to pairs[row * k ...].
template <int DT, int WAVES>
__device__ __forceinline__ void sort_and_store(const uint32_t* fk, const uint32_t* fi, uint32_t* xk, uint32_t* xi,
                                               uint64_t* xs, uint32_t k, void* out_vals, IdxOut out_idx,
                                               uint2* pairs, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  if (k <= 64u * kMaxRuns) {
    const uint32_t runs = (k + 63u) / 64u;
    if (runs <= 1)
      sort_runs_store<DT, WAVES, 1>(fk, fi, xs, k, out_vals, out_idx, pairs, row);
    else if (runs <= 2)
      sort_runs_store<DT, WAVES, 2>(fk, fi, xs, k, out_vals, out_idx, pairs, row);
    else if (runs <= 4)
      sort_runs_store<DT, WAVES, 4>(fk, fi, xs, k, out_vals, out_idx, pairs, row);
    else if (runs <= 8)
      sort_runs_store<DT, WAVES, 8>(fk, fi, xs, k, out_vals, out_idx, pairs, row);
    else
      sort_runs_store<DT, WAVES, 16>(fk, fi, xs, k, out_vals, out_idx, pairs, row);
    return;
  }
  uint32_t cap = 64;
  while (cap < k) cap <<= 1;
  if (cap > 8 * NT) {
    sort_store_lds<DT, WAVES>(fk, fi, xk, xi, k, cap, out_vals, out_idx, pairs, row);
    return;
  }
  switch (cap) {
    case 64: sort_store_t<DT, WAVES, 6>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row); break;
    case 128: sort_store_t<DT, WAVES, 7>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row); break;
    case 256: sort_store_t<DT, WAVES, 8>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row); break;
    case 512: sort_store_t<DT, WAVES, 9>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row); break;
    case 1024:
      if constexpr (1024 <= 8 * NT) sort_store_t<DT, WAVES, 10>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row);
      break;
    case 2048:
      if constexpr (2048 <= 8 * NT) sort_store_t<DT, WAVES, 11>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row);
      break;
    default:
      if constexpr (4096 <= 8 * NT) sort_store_t<DT, WAVES, 12>(fk, fi, xk, xi, k, out_vals, out_idx, pairs, row);
      break;
  }
}

// --------------------------------------------------------------------------- slice merge

// Where a list merge writes its k entries: outputs vals/idx from row offset at0, or pairs.
struct MergeOut {
  void* vals;
  IdxOut idx;
  uint2* pairs;
  uint64_t at0;
};

// Merge of S sorted lists (S <= MAXS <= kMaxListGroup, k entries each, best first, as
// (key, index) pairs at src[s * k + i]) into their k best, sorted: written to the outputs at
// at0 + rank, or, with pairs, as pairs at pairs[rank] (outs() gives them, a MergeOut; it is
// called once the lists are loaded). The lists are loaded into LDS as
// composites (lds: S * k 64-bit words, then S 32-bit prefix lengths); an entry's place in
// the merged order is its position in its own list plus, for every other list, the number
// of that list's entries that rank above it (binary searches, the other lists searched in
// the same step; equal entries of earlier lists count as above). Padding (composite 0)
// ranks below every element; it is placed only when the lists hold fewer than k elements
// together, as padding. Places the entries of lists [l0, l1) (all lists are loaded); each
// thread places EB entries at a time, their searches interleaved step by step (long lists:
// the searches' LDS round trips overlap).
template <int DT, int WAVES, uint32_t MAXS, uint32_t EB, class Outs>
__device__ __forceinline__ void merge_lists_t(const uint2* src, uint32_t S, uint32_t k, uint32_t pk, uint64_t* lds,
                                              Outs outs, uint32_t l0, uint32_t l1) {
  constexpr uint32_t NT = WAVES * 64, MO = MAXS - 1;  // MO: the other lists an entry searches
  const uint32_t tid = threadIdx.x, total = S * k;
  __attribute__((address_space(3))) uint64_t* lw = lds_ptr(lds);
  // fill: LU 16-byte loads (two entries each) in flight per thread before their LDS writes
  // (a plain loop waits for each load in turn); buffer loads past the lists read zeros
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint2*>(src), 0, static_cast<int>(total * 8u), kRsrcWord3);
  const uint32_t npair = (total + 1u) / 2u;
  auto fill = [&](auto lu) {
    constexpr uint32_t LU = decltype(lu)::value;
    for (uint32_t p0 = tid; p0 < npair; p0 += LU * NT) {
      u32x4 v[LU];
#pragma unroll
      for (uint32_t u = 0; u < LU; ++u) v[u] = load16(rs, (p0 + u * NT) * 16u);
#pragma unroll
      for (uint32_t u = 0; u < LU; ++u) {
        const uint32_t e = 2u * (p0 + u * NT);
        if (e < total) lw[e] = comp_of(v[u][0], v[u][1]);
        if (e + 1u < total) lw[e + 1u] = comp_of(v[u][2], v[u][3]);
      }
    }
  };
  if (npair <= 2u * NT)
    fill(std::integral_constant<uint32_t, 2>{});  // short lists: no loads wasted past the end
  else
    fill(std::integral_constant<uint32_t, 8>{});
  lds_sync();
  // the outputs: read now, their loads overlap the searches
  const MergeOut mo = outs();
  // Entries below T cannot reach the first k places, so they are not searched: one list's
  // k-th entry has k entries (its list's first k) at or above it, and each of the S lists
  // has ceil(k/S) entries at or above the smallest of the lists' ceil(k/S)-th entries; T is
  // the larger of the two bounds (broadcast LDS reads, the same in every thread).
  uint64_t ta = 0, tb = ~0ull;
#pragma unroll
  for (uint32_t q = 0; q < MAXS; ++q) {
    const uint32_t qq = min(q, S - 1u);
    const uint64_t a = lw[qq * k + k - 1u], b = lw[qq * k + pk - 1u];
    ta = a > ta ? a : ta;
    tb = b < tb ? b : tb;
  }
  const uint64_t T = ta > tb ? ta : tb;
  const uint32_t top = 1u << (31u - static_cast<uint32_t>(__builtin_clz(k)));  // largest power of two <= k
  // maxn: the longest of the lists' prefixes at or above T. Entries that rank above an entry
  // at or above T are themselves above T, so no count exceeds its list's prefix, and the
  // searches need only cover maxn places. Found for groups of 8 or more lists (for fewer,
  // the extra search and barrier cost more than they save).
  uint32_t top_n = top, maxn = k;
  if constexpr (MAXS >= 8) {
    __attribute__((address_space(3))) uint32_t* nql = lds_ptr(reinterpret_cast<uint32_t*>(lds + S * k));
    if (tid < S) {
      uint32_t n = 0;
      for (uint32_t step = top; step > 0; step >>= 1)
        n = (n + step <= k && lw[tid * k + n + step - 1u] >= T) ? n + step : n;
      nql[tid] = n;
    }
    lds_sync();
    maxn = 0;
#pragma unroll
    for (uint32_t q = 0; q < MAXS; ++q) maxn = max(maxn, q < S ? nql[q] : 0u);
    top_n = maxn ? 1u << (31u - static_cast<uint32_t>(__builtin_clz(maxn))) : 0u;
  }
  // The counts: every count is at most N (k, or the longest prefix); m is the largest power
  // of two <= N. A first probe at m - 1 leaves a window of m counts, [0, m) or [N - m + 1, N]
  // (a count of at least m is at least N - m + 1, as N < 2m), and binary steps m/2 ... 1 find
  // the count inside it (Shar's search for lengths that are not powers of two): every probe
  // lands inside its list, so the steps need no clamps. An entry's own list is not searched,
  // and a list before its own, whose equal entries rank above it, is searched for c - 1.
  const uint32_t N = maxn, m = top_n;
  const uint32_t e_end = l1 * k;
  for (uint32_t e0 = l0 * k + tid; e0 < e_end; e0 += EB * NT) {
    uint64_t c[EB], cq[EB][MO];
    uint32_t s[EB], ad[EB][MO];  // ad: LDS byte address of the list's first entry past the count
    bool act[EB];
#pragma unroll
    for (uint32_t b = 0; b < EB; ++b) {
      const uint32_t e = e0 + b * NT;
      s[b] = 0;
#pragma unroll
      for (uint32_t q = 1; q < MAXS; ++q) s[b] += (q < S && e >= q * k) ? 1u : 0u;
      c[b] = e < e_end ? lw[e] : 0ull;
      // entries below T are not placed, nor is padding past the first list: the earlier
      // lists' k entries rank above it
      act[b] = e < e_end && c[b] >= T && (c[b] != 0u || s[b] == 0u);
#pragma unroll
      for (uint32_t q = 0; q < MO; ++q) {
        const uint32_t oq = q < s[b] ? q : q + 1u;  // the q-th list other than the entry's own
        ad[b][q] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lw + min(oq, S - 1u) * k));
        cq[b][q] = q < s[b] && act[b] ? c[b] - 1u : c[b];
      }
    }
    // a list's entries at or above T are its first ones, so the waves past them have nothing
    // to place and skip the search
    bool any = false;
#pragma unroll
    for (uint32_t b = 0; b < EB; ++b) any = any || act[b];
    if (ballot(any) == 0) continue;
    auto at = [](uint32_t a) {
      return *reinterpret_cast<__attribute__((address_space(3))) const uint64_t*>(static_cast<uintptr_t>(a));
    };
    if (m > 0) {
      uint64_t x[EB][MO];
#pragma unroll
      for (uint32_t b = 0; b < EB; ++b)
#pragma unroll
        for (uint32_t q = 0; q < MO; ++q) x[b][q] = at(ad[b][q] + 8u * (m - 1u));
#pragma unroll
      for (uint32_t b = 0; b < EB; ++b)
#pragma unroll
        for (uint32_t q = 0; q < MO; ++q) ad[b][q] += x[b][q] > cq[b][q] ? 8u * (N - m + 1u) : 0u;
      for (uint32_t step = m >> 1; step > 0; step >>= 1) {
#pragma unroll
        for (uint32_t b = 0; b < EB; ++b)
#pragma unroll
          for (uint32_t q = 0; q < MO; ++q) x[b][q] = at(ad[b][q] + 8u * (step - 1u));
#pragma unroll
        for (uint32_t b = 0; b < EB; ++b)
#pragma unroll
          for (uint32_t q = 0; q < MO; ++q) ad[b][q] += x[b][q] > cq[b][q] ? 8u * step : 0u;
      }
    }
#pragma unroll
    for (uint32_t b = 0; b < EB; ++b) {
      uint32_t rank = e0 + b * NT - s[b] * k;
#pragma unroll
      for (uint32_t q = 0; q < MO; ++q) {
        const uint32_t oq = q < s[b] ? q : q + 1u;
        const uint32_t a0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lw + min(oq, S - 1u) * k));
        rank += oq < S ? (ad[b][q] - a0) / 8u : 0u;  // past the last list: a clamped copy, not counted
      }
      if (act[b] && rank < k) store_out<DT>(mo.vals, mo.idx, mo.pairs, mo.at0 + rank, c[b]);
    }
  }
}

// Integer compare values for the streaming filter, from the threshold pair (key, idx).
// mode 1: hit <=> (int)score > thr; mode 2: hit <=> score < thr; "strict" is used for
// blocks after the threshold's index, "non-strict" (ties win) for blocks before it.
// bf16 scores carry the element in the high 16 bits.
template <int DT>
__device__ __forceinline__ void filter_thresholds(uint32_t tkey, uint32_t& mode, uint32_t& thr_s, uint32_t& thr_n) {
  const uint32_t raw = raw_of_key<DT>(tkey);
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

// --------------------------------------------------------------------------- DeepSelect body
// Byte offset past every buffer range: a load there returns zeros and reads no memory.
constexpr uint32_t kNoLoad = 0x7FFFFFF0u;

// One workgroup runs DeepSelect over `len` items of a 16-byte-aligned stream (rs).
// MERGE == false: items are raw elements of type DT (the select kernel); MERGE == true:
// items are (key, index) pairs of 8 bytes (the merge kernel). Ends with the k survivors,
// unordered, in (*fk, *fi) (visible to every thread).
struct BodyOut {
  const uint32_t* fk;
  const uint32_t* fi;
  uint64_t reads, jsum;  // this thread's share of the elements read and of their indices
  bool sorted;           // the final compaction already wrote the sorted output
};

// Stream geometry of a DeepSelect body: items of IB bytes (raw elements, or 8-byte (key,
// index) pairs for the merge kernel), VEC per lane per 16-byte chunk, blocks of B items (each
// wave filters CPW chunks of every block).
template <int DT, int WAVES, int CPW, bool MERGE>
struct StreamGeom {
  static constexpr uint32_t IB = MERGE ? 8 : (DT == DS_BF16 ? 2 : 4);  // bytes per item
  static constexpr uint32_t VEC = 16 / IB;                            // items per lane per chunk
  static constexpr uint32_t CHUNK = 64 * VEC;
  static constexpr uint32_t B = WAVES * CPW * CHUNK;
  // byte offset of this lane's part of chunk t of block bid (no read for bid >= m)
  static __device__ __forceinline__ uint32_t offset(uint32_t bid, uint32_t t, uint32_t m, uint32_t wave,
                                                    uint32_t lane) {
    return bid < m ? (bid * B + (wave + t * WAVES) * CHUNK + lane * VEC) * IB : kNoLoad;
  }
};

// Block order: the permutation `ord` is over groups of 2^gshift consecutive blocks; the i-th
// block read is block (i mod 2^gshift) of group ord(i >> gshift). Positions past the last
// block (the last group's padding, or steps past the end, i >= m_iter) give the empty id m.
__device__ __forceinline__ uint32_t order_bid(const BlockOrder& ord, uint32_t i, uint32_t gshift, uint32_t m,
                                              uint32_t m_iter) {
  if (i >= m_iter) return m;
  const uint32_t b = (ord.at(i >> gshift) << gshift) | (i & ((1u << gshift) - 1u));
  return b < m ? b : m;
}

// The first D blocks of a stream's order: their ids and their loads in flight. A kernel
// requests them before the rest of its set-up (parameter reads from the argument block
// included), so that their latency overlaps all of it.
template <int D, int CPW>
struct FirstBlocks {
  u32x4 buf[D][CPW];
  uint32_t bids[D];
};

template <int DT, int WAVES, int CPW, int D, bool MERGE>
__device__ __forceinline__ void first_blocks(__amdgpu_buffer_rsrc_t rs, uint32_t len, const BlockOrder& ord,
                                             uint32_t gshift, FirstBlocks<D, CPW>& fb) {
  using G = StreamGeom<DT, WAVES, CPW, MERGE>;
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint32_t m = (len + G::B - 1) / G::B;
  const uint32_t m_iter = ((m + (1u << gshift) - 1u) >> gshift) << gshift;
  // lane l evaluates position l mod D in vector registers (see to_vgpr)
  const uint32_t first_bid = order_bid(ord, to_vgpr(0u) + lane % static_cast<uint32_t>(D), gshift, m, m_iter);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    fb.bids[d] = __builtin_amdgcn_readlane(first_bid, d);
#pragma unroll
    for (uint32_t t = 0; t < CPW; ++t) fb.buf[d][t] = load16(rs, G::offset(fb.bids[d], t, m, wave, lane));
  }
}

// Schedule. The design note checks the buffer once after each whole block ("lockstep":
// a workgroup barrier after every block, then the check). By default the waves instead
// stream independently: each wave filters its share of block after block, reserves buffer
// space with one LDS atomic, and checks the buffer length itself (from the atomic's
// return, or by reading it when it had no hits). A wave that sees the length at or past
// k + B2 stops at a barrier; the other waves stop there at their next check, and a wave
// that has no blocks left waits there. After the barrier every wave reads the same
// length, and they compact together (or, once every wave is done, run the final
// compaction). A wave appends at most one more share of a block after the length crosses
// k + B2 (it checks after every share), so the buffer never exceeds k + B2 + B - 1 entries,
// the design note's bound. The threshold only changes at compactions, so a wave always
// filters with the workgroup's current threshold.
//
// D buffers of CPW chunks per wave are in flight: block i+D is loaded into the registers of
// block i as soon as block i has been filtered. The loop body handles D blocks with D
// separate buffers and has no exit, so the compiler sees which loads are the older ones and
// waits only for those.
template <int DT, int WAVES, int CPW, int D, bool MERGE, bool STATS>
__device__ __forceinline__ void deepselect_body(const Lay& L, Scalars& sc, __amdgpu_buffer_rsrc_t rs, uint32_t len,
                                                uint32_t idx_base, uint32_t k, uint32_t B2, const BlockOrder& ord,
                                                uint32_t ilo, uint32_t ihi, bool lockstep, uint32_t warm,
                                                unsigned long long* share, bool presample, uint32_t gshift,
                                                FirstBlocks<D, CPW>& fb, const OutSpec* fso, BodyOut& out) {
  using G = StreamGeom<DT, WAVES, CPW, MERGE>;
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t VEC = G::VEC, CHUNK = G::CHUNK, B = G::B;
  constexpr uint32_t SHARE = CPW * CHUNK;  // items of one block that one wave filters
  constexpr uint32_t key_hi = DT == DS_BF16 ? 0xFFFFu : 0xFFFFFFFFu;  // largest possible key
  static_assert(D >= 2 && D <= 4, "two to four buffers");
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wave_s = uni(wave);  // the same, known to the compiler as uniform
  // LDS byte addresses of the append buffer, of this lane's dummy slot, and the distance from
  // a key slot to its index slot
  const uint32_t ck_addr = lds_addr(L.ck), dummy_addr = ck_addr + 4u * (L.dummy + lane);
  const uint32_t ci_off = lds_addr(L.ci) - ck_addr;
  const uint32_t m = (len + B - 1) / B;

  // Block order (order_bid): ng groups of 2^gshift blocks. The group order is a table for up
  // to kOrdCap groups, computed on the fly beyond.
  const uint32_t ng = (m + (1u << gshift) - 1u) >> gshift, m_iter = ng << gshift;
  // (a stream of at most D blocks reads only the first D ids, computed directly: no table)
  const bool tab = ng <= kOrdCap && m_iter > static_cast<uint32_t>(D);
  // block id of the i-th block read, from the permutation itself (direct) or its table
  // (the table's first 64 entries are also held in a vector register, lane l entry l, once
  // it is built: a lookup there is a lane read, with no LDS access queued behind the appends)
  uint32_t ordv = 0;
  auto bid_of = [&](uint32_t i) -> uint32_t {
    if (i >= m_iter) return m;
    const uint32_t g = i >> gshift;
    const uint32_t o = !tab ? ord.at(g) : (g < 64u ? __builtin_amdgcn_readlane(ordv, g) : uni(L.ordt[g]));
    const uint32_t b = (o << gshift) | (i & ((1u << gshift) - 1u));
    return b < m ? b : m;
  };

  // threshold state (uniform across the workgroup; it changes only at compactions)
  uint32_t mode = 0, thr_s = ~0u, thr_n = ~0u;  // mode 0: accept everything (no threshold yet)
  uint32_t t_key = 0, t_idx = 0, maxkey = 0;
  uint32_t f_idx = 0;  // the filter's index threshold (its key threshold is in thr_s / thr_n)
  uint32_t nsurv = 0, hpar = 0;
  uint32_t warm_left = warm;  // blocks of the warm-up window still to come
  bool sur_a = false;  // survivors in set A (else set B)
  // key range of the entries appended before the first compaction (the select kernel tracks
  // it; the merge kernel does not)
  uint32_t rmin_w = ~0u, rmax_w = 0;
  constexpr bool range_ok = !MERGE;
  // presampled threshold (a lower bound of the first block's k-th element) and the first
  // block's largest key, the value-bin window of the first compaction
  bool presampled = false;
  uint32_t pre_hi = 0;
  [[maybe_unused]] const bool st0 = STATS && tid == 0;  // the thread that keeps the counters in sc.st_*
  [[maybe_unused]] uint64_t t_mark = 0;
  uint64_t my_reads = 0, my_jsum = 0;

  auto addr = [&](uint32_t bid, uint32_t t) -> uint32_t { return G::offset(bid, t, m, wave, lane); };

  // The first D blocks were requested by the kernel (first_blocks) before anything else, so
  // their latency overlaps the set-up below (their ids come from the permutation directly,
  // the rest from its table).
  auto& buf = fb.buf;
  auto& bids = fb.bids;

  // workgroup state: histograms, counters, the order table
  for (uint32_t i = 4u * tid; i < 2u * kBins; i += 4u * NT) *reinterpret_cast<uint4*>(L.hist + i) = make_uint4(0, 0, 0, 0);
  if (tid == 0) {
    sc.len = 0;
    sc.done = 0;
    sc.st_p = 0;
    if constexpr (STATS) {
      sc.st_a = sc.st_r = sc.st_w = sc.st_max = sc.st_tc = sc.st_ts = sc.st_tf = 0;
      sc.st_mono = 1;
      sc.reads = 0;
      sc.index_sum = 0;
    }
    if (share) {  // what the row's other slices have published so far
      const uint64_t g = __hip_atomic_load(share, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sc.shr[0] = static_cast<uint32_t>(g);
      sc.shr[1] = static_cast<uint32_t>(g >> 32);
    }
  }
  if (tab)
    for (uint32_t i = tid; i < ng; i += NT) L.ordt[i] = ord.at(i);
  lds_sync();
  if (tab) ordv = L.ordt[lane];  // entries past ng are never read back
  if (share && (sc.shr[0] | sc.shr[1]) != 0) {
    // filter with the row's threshold from the start (no own threshold yet)
    f_idx = ~sc.shr[0];
    filter_thresholds<DT>(sc.shr[1], mode, thr_s, thr_n);
  }

  bool sorted = false;
  // A compaction of the nsurv survivors and the napp entries appended since the last one.
  // In-loop calls clear the append counter before their last barrier, so no wave can
  // append before it is cleared.
  auto compaction = [&](uint32_t napp, bool fin) {
    const Segs sg = nsurv ? make_segs(sur_a ? L.ck : L.bk, sur_a ? L.ci : L.bi, nsurv, L.ck + L.k4, L.ci + L.k4, napp)
                          : make_segs(nullptr, nullptr, 0u, L.ck, L.ci, napp);
    const bool to_a = nsurv != 0 && !sur_a;  // first compaction: entries start in A, go to B
    // value bins over [T, previous maximum], or over the appended keys' range the first time
    uint32_t vlo = t_key, vhi = maxkey;
    bool vok = nsurv != 0;
    if (!nsurv && presampled) {
      vhi = pre_hi;
      vok = true;
    } else if (!nsurv) {
      vlo = ~0u;
      vhi = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        vlo = min(vlo, sc.rmin[w]);
        vhi = max(vhi, sc.rmax[w]);
      }
      vok = range_ok;
    }
    if constexpr (STATS) {
      if (st0) {
        sc.st_a += napp;
        sc.st_w += nsurv + napp;
        sc.st_max = max(sc.st_max, static_cast<unsigned long long>(nsurv + napp));
      }
    }
    compact<WAVES, DT, !MERGE>(sg, to_a ? L.ck : L.bk, to_a ? L.ci : L.bi, k, fin, nsurv != 0, key_hi, ilo, ihi, sc,
                               L.hist, hpar, t_key, t_idx, maxkey, vlo, vhi, vok, fin ? fso : nullptr, sorted,
                               fin ? nullptr : &sc.len, reinterpret_cast<uint64_t*>(L.ck));
    sur_a = to_a;
  };

  // In-loop compaction (every wave calls it at the same barrier count), then the new filter.
  // The filter's threshold: the slice's own (T0 or the last compaction's k-th entry), or, with
  // a shared row threshold, the larger of it and the row's. The slice publishes its own to
  // the row's word with an atomic maximum and reads back what the row's slices published so
  // far. Every published value ranks at or below the row's k-th element (a slice's k-th best
  // so far, or a lower bound of it), so filtering with it drops nothing of the row's top k;
  // compactions keep the slice's own threshold (the buffer may hold entries below the row's).
  auto set_filter = [&]() {
    uint32_t fk = t_key, fi = t_idx;
    if (share) {
      if (tid == 0) {
        const uint64_t old =
            __hip_atomic_fetch_max(share, static_cast<unsigned long long>(comp_of(t_key, t_idx)), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        sc.shr[0] = static_cast<uint32_t>(old);
        sc.shr[1] = static_cast<uint32_t>(old >> 32);
      }
      lds_sync();
      const uint64_t g = (static_cast<uint64_t>(sc.shr[1]) << 32) | sc.shr[0];
      if (g > comp_of(fk, fi)) {
        fk = static_cast<uint32_t>(g >> 32);
        fi = ~static_cast<uint32_t>(g);
      }
    }
    f_idx = fi;
    filter_thresholds<DT>(fk, mode, thr_s, thr_n);
  };

  auto in_loop = [&](uint32_t napp) {
    [[maybe_unused]] const uint64_t prev_c = comp_of(t_key, t_idx);
    [[maybe_unused]] const bool had_t = nsurv != 0;
    if constexpr (STATS) {
      if (st0) t_mark = wall_clock64();
    }
    compaction(napp, false);
    if constexpr (STATS) {
      if (st0) {
        sc.st_tc += wall_clock64() - t_mark;
        sc.st_r += 1;
        if (had_t && comp_of(t_key, t_idx) < prev_c) sc.st_mono = 0;
      }
    }
    nsurv = k;
    if constexpr (!MERGE)
      set_filter();
    else
      mode = 1;
  };

  // The stop of a free-running wave that saw the buffer at or past k + B2: one barrier, then
  // the compaction every other wave joins (the length cannot shrink before it).
  auto stop_and_compact = [&]() {
    if constexpr (STATS) {
      if (st0) t_mark = wall_clock64();
    }
    lds_sync();
    if constexpr (STATS) {
      if (st0) sc.st_ts += wall_clock64() - t_mark;
    }
    in_loop(sc.len);
  };

  // Threshold from the first (whole) block instead of "accept everything", from each lane's
  // largest key lmax (over elements of the stream, each lane its own): each wave takes the
  // j-th largest of its lanes' maxima, j = ceil(k / WAVES), found bit by bit over the key's
  // top 16 bits (a truncation can only lower it); the smallest of the waves' values T0 has
  // at least WAVES * j >= k distinct elements (one per lane) at or above it, so T0 does not
  // exceed the k-th element and "key >= T0" keeps every element that can be in the top k.
  auto presample_from = [&](uint32_t lmax) {
    constexpr uint32_t KB = DT == DS_BF16 ? 16u : 32u;
    const uint32_t j = (k + WAVES - 1) / WAVES;
    uint32_t pre = 0;
#pragma unroll
    for (uint32_t b = KB; b > KB - 16u; --b) {
      const uint32_t cand = pre | (1u << (b - 1u));
      pre = popc(ballot(lmax >= cand)) >= j ? cand : pre;
    }
    const uint32_t wmax = wave_max32(lmax);
    if (lane == 0) {
      sc.rmin[wave] = pre;
      sc.rmax[wave] = wmax;
    }
    lds_sync();
    uint32_t t0 = ~0u, hi = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      t0 = min(t0, sc.rmin[w]);
      hi = max(hi, sc.rmax[w]);
    }
    t_key = t0;
    t_idx = ~0u;  // ties with T0 are kept in every block
    pre_hi = hi;
    presampled = true;
    mode = 1;
  };

  // Reserves `cnt` buffer entries for this wave (one LDS atomic); returns the first slot
  // (relative to the append region) and the length after this reservation in `seen`.
  auto reserve = [&](uint32_t cnt, uint32_t& seen) -> uint32_t {
    uint32_t pos = 0;
    if (lane == 0) pos = atomicAdd(&sc.len, cnt);
    pos = uni(pos);
    seen = pos + cnt;
    return pos;
  };

  // Filter block `bid` (the i-th in the order) from `buf`, refill `buf` with block i+D, and
  // check the buffer.
  auto process = [&](u32x4(&bf)[CPW], uint32_t& bid_ref, uint32_t i) {
    const uint32_t bid = bid_ref;
    const uint32_t blk_lo = bid * B;
    // the id of block i+D, read now: read after the filter's LDS stores, its wait would also
    // wait for those stores and hold back the refill
    const uint32_t next_bid = bid_of(i + D);
    const uint32_t app0 = nsurv ? L.k4 : 0u;  // the append region
    // The stream length as a value the optimizer cannot reason about: with the counters
    // compiled in, clang (ROCm 7.2) dropped the length check of all but the last chunk of a
    // share, so zero padding past the end was appended (measured); an empty asm on the
    // uniform value keeps every check.
    uint32_t len_opaque = len;
    asm volatile("" : "+s"(len_opaque));
    uint32_t seen = 0;                        // buffer length after this wave's last reservation
    bool reserved = false;
    if constexpr (!MERGE) {
      uint32_t s[CPW][VEC];  // the block's scores (bf16: the element in bits 16-31)
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) {
        if constexpr (DT == DS_BF16) {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) {
            s[t][2 * q] = bf[t][q] << 16;
            s[t][2 * q + 1] = bf[t][q];
          }
        } else {
#pragma unroll
          for (uint32_t q = 0; q < 4; ++q) s[t][q] = bf[t][q];
        }
      }
      if constexpr (STATS) {
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) {
          const uint32_t first = blk_lo + (wave + t * WAVES) * CHUNK + lane * VEC;
          const uint32_t nval = first >= len ? 0u : min(VEC, len - first);
          my_reads += nval;
          my_jsum += nval * static_cast<uint64_t>(idx_base + first) + (static_cast<uint64_t>(nval) * (nval - 1)) / 2;
        }
      }
      if (presample && i == 0 && blk_lo + B <= len) {
        // each lane's maximum over its elements of this block and of every other whole block
        // already in flight (the next D - 1 of the order): all of them were requested at the
        // start and arrive together, and more elements give a tighter T0
        uint32_t lmax = 0;
        if constexpr (DT == DS_BF16) {
          // two keys per word, with packed 16-bit operations (a bf16's key is its bits with
          // the sign bit flipped, or all of them for a negative value)
          using u16x2 = uint16_t __attribute__((ext_vector_type(2)));
          using i16x2 = int16_t __attribute__((ext_vector_type(2)));
          u16x2 acc = {0, 0};
          auto fold = [&](uint32_t w) {
            const u16x2 x = __builtin_bit_cast(u16x2, w);
            const u16x2 neg = __builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, x) >> 15);
            acc = __builtin_elementwise_max(acc, x ^ (neg | static_cast<uint16_t>(0x8000u)));
          };
#pragma unroll
          for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) fold(bf[t][q]);
          }
#pragma unroll
          for (int d = 1; d < D; ++d) {
            if (bids[d] < m && bids[d] * B + B <= len) {
#pragma unroll
              for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
                for (uint32_t q = 0; q < 4; ++q) fold(buf[d][t][q]);
              }
            }
          }
          lmax = max(static_cast<uint32_t>(acc.x), static_cast<uint32_t>(acc.y));
        } else {
#pragma unroll
          for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
            for (uint32_t q = 0; q < VEC; ++q) lmax = max(lmax, key_of_score<DT>(s[t][q]));
          }
#pragma unroll
          for (int d = 1; d < D; ++d) {
            if (bids[d] < m && bids[d] * B + B <= len) {
#pragma unroll
              for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
                for (uint32_t q = 0; q < 4; ++q) lmax = max(lmax, key_of_score<DT>(buf[d][t][q]));
              }
            }
          }
        }
        presample_from(lmax);
        set_filter();
      }
      const bool strict = idx_base + blk_lo > f_idx;
      const uint32_t thr = strict ? thr_s : thr_n;
      // The hits of the block, appended raw. ONE: a positive threshold (mode 1), compiled on
      // its own so that the hit masks are never merged across the modes' branches.
      auto filter_hits = [&](auto one) {
        constexpr bool ONE = decltype(one)::value;
        // a score that never passes this mode's compare (for the stream's tail)
        constexpr uint32_t NEVER = ONE ? 0x80000000u : 0xFFFFFFFFu;
        uint32_t kmn = ~0u, kmx = 0;  // key range of the hits while there is no threshold
        // One reservation per chunk: only that chunk's hit masks are live. Hits are stored raw;
        // a lane without a hit in an element that some lane of the wave hit writes its dummy
        // slot instead, so the stores need no exec-mask changes.
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) {
          const uint32_t cfirst = blk_lo + (wave_s + t * WAVES) * CHUNK;  // the chunk's first element
          const uint32_t first = cfirst + lane * VEC;
          if (cfirst + CHUNK > len_opaque) {  // the stream's tail chunk, or a chunk past its end
#pragma unroll
            for (uint32_t e = 0; e < VEC; ++e) s[t][e] = first + e < len_opaque ? s[t][e] : NEVER;
          }
          // the hit masks are computed once, on straight-line code (no mask merging)
          bool h[VEC];
#pragma unroll
          for (uint32_t e = 0; e < VEC; ++e) {
            if constexpr (ONE)
              h[e] = static_cast<int32_t>(s[t][e]) > static_cast<int32_t>(thr);
            else  // mode 2, or mode 0 (thr ~0: every non-NaN score passes)
              h[e] = s[t][e] < thr;
          }
          if (!ONE && mode == 0) {
#pragma unroll
            for (uint32_t e = 0; e < VEC; ++e) {
              const uint32_t key = key_of_score<DT>(s[t][e]);
              kmn = h[e] ? min(kmn, key) : kmn;
              kmx = h[e] ? max(kmx, key) : kmx;
            }
          }
          // positions by vector arithmetic only (the CU's waves share one scalar unit): the
          // lane's hit count, its exclusive prefix over the wave, one reservation; every
          // element then goes to its slot or, if it is no hit, to the lane's dummy slot
          // (counted in bytes, 4 a hit, so that one value is both the count and the step of
          // the slot address)
          uint32_t hb[VEC], cnt = 0;  // hb: 4 for a hit
#pragma unroll
          for (uint32_t e = 0; e < VEC; ++e) {
            hb[e] = h[e] ? 4u : 0u;
            cnt += hb[e];
          }
          const uint32_t incl = wave_incl_scan(cnt);
          const uint32_t tot = __builtin_amdgcn_readlane(incl, 63) >> 2;
          if (tot) {
            // byte addresses: the key slot (the next free one, or the dummy), the index slot
            // at a fixed distance from it
            uint32_t pa = ck_addr + 4u * (app0 + reserve(tot, seen)) + incl - cnt;
            reserved = true;
            const uint32_t j0 = idx_base + first;
#pragma unroll
            for (uint32_t e = 0; e < VEC; ++e) {
              const uint32_t a = h[e] ? pa : dummy_addr;
              *lds_at(a) = s[t][e];
              *lds_at(a + ci_off) = j0 + e;
              pa += hb[e];
            }
          }
        }
        if (!ONE && mode == 0) {
          rmin_w = min(rmin_w, wave_min32(kmn));
          rmax_w = max(rmax_w, wave_max32(kmx));
          if (lane == 0) {
            sc.rmin[wave] = rmin_w;
            sc.rmax[wave] = rmax_w;
          }
        }
      };
      if (mode == 0 && blk_lo + B <= len) {
        // accept everything: each wave stores its chunks (raw) contiguously
        const uint32_t pos = app0 + reserve(SHARE, seen);
        reserved = true;
        uint32_t kmn = ~0u, kmx = 0;
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
          for (uint32_t q = 0; q < VEC; ++q) {
            const uint32_t key = key_of_score<DT>(s[t][q]);
            kmn = min(kmn, key);
            kmx = max(kmx, key);
          }
        }
        rmin_w = min(rmin_w, wave_min32(kmn));
        rmax_w = max(rmax_w, wave_max32(kmx));
        if (lane == 0) {
          sc.rmin[wave] = rmin_w;
          sc.rmax[wave] = rmax_w;
        }
        if (pos % 4u == 0) {
#pragma unroll
          for (uint32_t t = 0; t < CPW; ++t) {
            const uint32_t at = pos + t * CHUNK + lane * VEC;
            const uint32_t j0 = idx_base + blk_lo + (wave + t * WAVES) * CHUNK + lane * VEC;
#pragma unroll
            for (uint32_t q = 0; q < VEC; q += 4) {
              *reinterpret_cast<uint4*>(L.ck + at + q) = make_uint4(s[t][q], s[t][q + 1], s[t][q + 2], s[t][q + 3]);
              *reinterpret_cast<uint4*>(L.ci + at + q) = make_uint4(j0 + q, j0 + q + 1, j0 + q + 2, j0 + q + 3);
            }
          }
        } else {
#pragma unroll
          for (uint32_t t = 0; t < CPW; ++t) {
            const uint32_t at = pos + t * CHUNK + lane * VEC;
            const uint32_t j0 = idx_base + blk_lo + (wave + t * WAVES) * CHUNK + lane * VEC;
#pragma unroll
            for (uint32_t q = 0; q < VEC; ++q) {
              L.ck[at + q] = s[t][q];
              L.ci[at + q] = j0 + q;
            }
          }
        }
      } else if (mode == 1) {
        filter_hits(std::true_type{});
      } else {
        filter_hits(std::false_type{});
      }
    } else {
      if (presample && i == 0 && blk_lo + B <= len) {
        uint32_t lmax = 0;  // every item of a whole block is real
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) lmax = max(lmax, max(bf[t][0], bf[t][2]));
        presample_from(lmax);
      }
      // merge: items are (key, index) pairs; a hit beats T in the composite order
      bool h[CPW][2];
      uint64_t mk[CPW][2];
      uint32_t tot = 0;
#pragma unroll
      for (uint32_t t = 0; t < CPW; ++t) {
        const uint32_t first = blk_lo + (wave + t * WAVES) * CHUNK + lane * 2;
#pragma unroll
        for (uint32_t e = 0; e < 2; ++e) {
          const uint32_t key = bf[t][2 * e], id = bf[t][2 * e + 1];
          const bool beats = mode == 0 || key > t_key || (key == t_key && id < t_idx);
          h[t][e] = beats && first + e < len_opaque;
          mk[t][e] = ballot(h[t][e]);
          tot += popc(mk[t][e]);
        }
      }
      if (tot) {
        uint32_t pos = app0 + reserve(tot, seen);
        reserved = true;
#pragma unroll
        for (uint32_t t = 0; t < CPW; ++t) {
#pragma unroll
          for (uint32_t e = 0; e < 2; ++e) {
            if (mk[t][e]) {
              const uint32_t q = mbcnt(mk[t][e], pos);
              if (h[t][e]) {
                L.ck[q] = bf[t][2 * e];
                L.ci[q] = bf[t][2 * e + 1];
              }
              pos += popc(mk[t][e]);
            }
          }
        }
      }
    }

    // refill this buffer with block i+D (blocks i+1 .. i+D-1 are already in flight)
    bid_ref = next_bid;
#pragma unroll
    for (uint32_t t = 0; t < CPW; ++t) bf[t] = load16(rs, addr(bid_ref, t));

    // the warm-up window: the first `warm` blocks of the order (the last group's padding
    // step does not count)
    const bool in_window = warm_left != 0;
    if (bid < m && warm_left != 0) --warm_left;
    if (lockstep || in_window) {
      // the design note's schedule: every wave has appended its share of the block, then the
      // check; a second barrier keeps the length still until every wave has read it. The
      // warm-up window's blocks run this way too, and after its last one the buffer is
      // compacted as soon as it holds more than k entries: T is then the k-th best of the
      // window's elements
      if constexpr (STATS) {
        if (st0) t_mark = wall_clock64();
      }
      lds_sync();
      if constexpr (STATS) {
        if (st0) sc.st_ts += wall_clock64() - t_mark;
      }
      const uint32_t napp = sc.len;
      if constexpr (STATS) {
        if (st0) sc.st_max = max(sc.st_max, static_cast<unsigned long long>(nsurv + napp));
      }
      if (nsurv + napp >= k + B2 || (in_window && warm_left == 0 && nsurv + napp > k))
        in_loop(napp);
      else
        lds_sync();
    } else {
      if (!reserved) seen = uni(__atomic_load_n(lds_ptr(&sc.len), __ATOMIC_RELAXED));
      if (nsurv + seen >= k + B2) stop_and_compact();
    }
  };

  // Steps past the last block use the empty block id m: no loads, no hits, no effect.
  for (uint32_t i = 0; i < m_iter; i += D) {
    process(buf[0], bids[0], i);
    process(buf[1], bids[1], i + 1);
    if constexpr (D >= 3) process(buf[2], bids[2], i + 2);
    if constexpr (D >= 4) process(buf[3], bids[3], i + 3);
  }

  // The end of this wave's stream. Free-running waves wait until every wave is done; a
  // wave that stopped for a compaction meanwhile brings the others into it.
  uint32_t napp;
  if (lockstep) {
    napp = sc.len;  // every append happened before the last barrier
  } else {
    if (lane == 0) atomicAdd(&sc.done, 1u);
    for (;;) {
      lds_sync();
      napp = sc.len;
      if (sc.done == WAVES) break;
      in_loop(napp);
    }
  }

  // final compaction
  if constexpr (STATS) {
    if (st0) sc.st_tf = wall_clock64();
  }
  compaction(napp, true);
  out.fk = sur_a ? L.ck : L.bk;
  out.fi = sur_a ? L.ci : L.bi;
  out.reads = my_reads;
  out.jsum = my_jsum;
  out.sorted = sorted;
}

// --------------------------------------------------------------------------- select kernel
// The parameter block P at byte offset OFF of the kernel's argument segment, through a
// pointer the compiler cannot trace back to the segment: reads of it are issued where the
// code reads them, never hoisted above earlier code.
template <class P, uint32_t OFF>
__device__ __forceinline__ const P& params_after_loads() {
  using KPtr = const __attribute__((address_space(4))) uint8_t*;
  KPtr a = (KPtr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(a));
  return *(const P*)(a + OFF);
}

// Byte offset of select_kernel's parameter block in its argument segment: the arguments
// before it, each at its natural alignment (the AMDGPU kernel argument layout), take 64
// bytes (five 8-byte values, three int32, padding to 8, the lengths pointer). The kernel's
// signature and this offset change together.
constexpr uint32_t align_to(uint32_t v, uint32_t a) { return (v + a - 1u) / a * a; }
constexpr uint32_t kSelectParamsOffset =
    align_to(align_to(5u * 8u + 3u * 4u, alignof(const int32_t*)) + sizeof(const int32_t*), alignof(SelectParams));
static_assert(kSelectParamsOffset == 64u, "select_kernel argument layout");

// Byte offset of merge_lists_kernel's parameter block: a pointer, two 8-byte values and eight
// int32 before it take 56 bytes. The kernel's signature and this offset change together.
constexpr uint32_t kMergeParamsOffset = align_to(3u * 8u + 8u * 4u, alignof(MergeParams));
static_assert(kMergeParamsOffset == 56u, "merge_lists_kernel argument layout");
// EXT: the instantiation that serves ragged rows, the warm-up window and the shared row
// threshold; the plain one (EXT = false) has none of their code. The parameters the first
// loads depend on come as scalars ahead of the rest, so that the hardware can preload them
// into scalar registers at wave launch (14 dwords, up to the row count) instead of the waves
// waiting on a load of the argument block.
template <int DT, int WAVES, int CPW, bool STATS, bool EXT>
__global__ __launch_bounds__(WAVES * 64) void select_kernel(const uint8_t* px, int64_t pstride, int64_t pn, int64_t pslice_len,
                                                                  uint64_t pseed, int32_t pslices, int32_t pgshift,
                                                                  int32_t prows, const int32_t* plens,
                                                                  [[maybe_unused]] SelectParams p) {
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t EB = DT == DS_BF16 ? 2 : 4;
  constexpr uint32_t B = WAVES * CPW * 64 * (16 / EB);

  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ Scalars sc;

  const uint32_t tid = threadIdx.x;
  // a row's slices run on one XCD, where the merge of their lists reads them from L2
  uint32_t row, slice;
  xcd_unit(blockIdx.x, static_cast<uint32_t>(pslices), static_cast<uint32_t>(prows), row, slice);
  const uint32_t slice_lo = slice * static_cast<uint32_t>(pslice_len);
  int64_t n_row = pn;  // this row's length
  if constexpr (EXT) {
    if (plens) {
      const int64_t l = plens[row];
      n_row = l < 0 ? 0 : (l < n_row ? l : n_row);
    }
  }
  const int64_t rest = n_row - static_cast<int64_t>(slice_lo);
  const uint32_t len = rest <= 0 ? 0u : static_cast<uint32_t>(min(pslice_len, rest));
  const uint32_t m = (len + B - 1) / B;
  constexpr int D = depth_for(WAVES, CPW);
  [[maybe_unused]] uint64_t t_start = 0;
  if constexpr (STATS) t_start = wall_clock64();

  if (EXT && len == 0) {
    // a slice past its row's end (ragged rows): its k entries are all padding, which ranks
    // below every element (the row's outputs past its length read index -1)
    const uint32_t k = static_cast<uint32_t>(p.k);
    if (pslices == 1) {
      for (uint32_t i = tid; i < k; i += NT) store_out<DT>(p.out_vals, p.out_idx, nullptr, static_cast<uint64_t>(row) * k + i, 0ull);
    } else {
      uint2* const dst = p.ws + static_cast<uint64_t>(row) * p.ws_row_entries + static_cast<uint64_t>(slice) * k;
      for (uint32_t i = tid; i < k; i += NT) dst[i] = make_uint2(0u, kSentinelIdx);
    }
    if constexpr (STATS) {
      if (tid == 0) {
        ds_stats* o = p.stats + (row * static_cast<uint32_t>(pslices) + slice);
        *o = ds_stats{};
        o->monotone = 1;
        o->slice_lo = slice_lo;
        o->block = B;
        o->slack = static_cast<uint32_t>(p.slack);
      }
    }
    return;
  }

  const uint8_t* base = px + static_cast<uint64_t>(row) * pstride + static_cast<uint64_t>(slice_lo) * EB;
  // Range = the slice rounded up to whole 16-byte chunks: the hardware checks whole dwords, so
  // an exact byte count would zero the dword that holds a bf16 row's odd last element. Row
  // starts are 16-byte aligned, so the rounded range never leaves the row's last chunk.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(base), 0, static_cast<int>((len * EB + 15u) & ~15u), kRsrcWord3);
  const uint32_t gshift = static_cast<uint32_t>(pgshift);
  BlockOrder ord;
  ord.init(pseed, row, slice, (m + (1u << gshift) - 1u) >> gshift);
  FirstBlocks<D, CPW> fb;
  first_blocks<DT, WAVES, CPW, D, false>(rs, len, ord, gshift, fb);

  // The rest of the parameters come from the argument block in memory (the preloaded ones
  // end with the row count). They are read through a pointer the compiler cannot see
  // through, so that their loads are issued after the first block loads and their latency
  // overlaps those (hoisted to the top, the loads' waits came first: register spills of the
  // loaded values wait for them).
  const SelectParams& q = params_after_loads<SelectParams, kSelectParamsOffset>();
  const uint32_t k = static_cast<uint32_t>(q.k);
  const uint32_t B2 = static_cast<uint32_t>(q.slack);
  const Lay L = lay_of(lds, k, B2, B);

  // the final compaction writes the sorted output itself when it can: the row's outputs, or
  // the slice's sorted list for the list merge
  OutSpec fso{q.out_vals, IdxOut{q.out_idx.p, q.out_idx.wide}, nullptr, row};  // (field by field: in registers)
  if (pslices > 1)
    fso = OutSpec{nullptr, IdxOut{nullptr, 0}, q.ws + static_cast<uint64_t>(row) * q.ws_row_entries + slice * k, 0};
  fso.on = pslices == 1 || q.sorted_lists;

  BodyOut bo;
  deepselect_body<DT, WAVES, CPW, D, false, STATS>(L, sc, rs, len, slice_lo, k, B2, ord, slice_lo, slice_lo + len - 1u,
                                                q.lockstep != 0, EXT ? static_cast<uint32_t>(q.warmup) : 0u,
                                                EXT && q.share ? q.share + row : nullptr, q.presample != 0, gshift,
                                                fb, &fso, bo);

  if constexpr (STATS) {
    const uint32_t lane = tid & 63u;
    uint64_t my_reads = bo.reads, my_jsum = bo.jsum;
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
      ds_stats* o = q.stats + (row * static_cast<uint32_t>(pslices) + slice);
      o->appended = sc.st_a;
      o->compactions = sc.st_r;
      o->work = sc.st_w;
      o->max_len = sc.st_max;
      o->reads = sc.reads;
      o->index_sum = sc.index_sum;
      o->monotone = sc.st_mono;
      o->slice_lo = slice_lo;
      o->slice_len = len;
      o->block = B;
      o->slack = B2;
      o->t_compact_ns = sc.st_tc * 10;
      o->t_sync_ns = sc.st_ts * 10;
      o->passes = sc.st_p;
    }
  }

  if (bo.sorted) {
    // done by the final compaction
  } else if (pslices == 1 && q.unsorted) {
    // the k survivors as the final compaction left them (no sort)
    for (uint32_t i = tid; i < k; i += NT)
      store_out<DT>(q.out_vals, q.out_idx, nullptr, static_cast<uint64_t>(row) * k + i, comp_of(bo.fk[i], bo.fi[i]));
  } else if (pslices == 1) {
    sort_and_store<DT, WAVES>(bo.fk, bo.fi, L.ck + L.k4, L.ci + L.k4, reinterpret_cast<uint64_t*>(L.hist), k,
                              q.out_vals, q.out_idx, nullptr, row);
  } else if (!q.sorted_lists) {
    uint2* const dst = q.ws + static_cast<uint64_t>(row) * q.ws_row_entries + static_cast<uint64_t>(slice) * k;
    for (uint32_t i = tid; i < k; i += NT) dst[i] = make_uint2(bo.fk[i], bo.fi[i]);
  } else {
    // the list-merge kernel merges the slices' sorted lists
    uint2* const rws = q.ws + static_cast<uint64_t>(row) * q.ws_row_entries;
    sort_and_store<DT, WAVES>(bo.fk, bo.fi, L.ck + L.k4, L.ci + L.k4, reinterpret_cast<uint64_t*>(L.hist), k, nullptr,
                              IdxOut{nullptr, 0}, rws + slice * k, 0);
  }
  if constexpr (STATS) {
    if (tid == 0) {
      const uint64_t t_end = wall_clock64();
      ds_stats* o = q.stats + (row * static_cast<uint32_t>(pslices) + slice);
      o->t_total_ns = (t_end - t_start) * 10;
      o->t_final_ns = (t_end - sc.st_tf) * 10;
    }
  }
}

// --------------------------------------------------------------------------- merge kernel
// DeepSelect again, over the slices' survivors of one row: items are (key, index) pairs.
template <int DT, int WAVES, int CPW>
__global__ __launch_bounds__(WAVES * 64) void merge_kernel(MergeParams p) {
  constexpr uint32_t NT = WAVES * 64;
  constexpr uint32_t B = WAVES * CPW * 128;

  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  __shared__ Scalars sc;

  const uint32_t tid = threadIdx.x;
  const uint32_t row = blockIdx.x;
  const uint32_t len = static_cast<uint32_t>(p.entries);
  const uint32_t m = (len + B - 1) / B;
  const uint32_t k = static_cast<uint32_t>(p.k);
  const uint32_t B2 = static_cast<uint32_t>(p.slack);

  const Lay L = lay_of(lds, k, B2, B);
  const uint2* base = p.ws + static_cast<uint64_t>(row) * p.row_entries;  // rows padded to 16 bytes
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint2*>(base), 0, static_cast<int>((len * 8u + 15u) & ~15u), kRsrcWord3);
  if (p.lens) {
    // A ragged row shorter than k: every one of its elements survived in its slice (the
    // first entries of each slice's list, the rest padding), so they are gathered, padded
    // to k and sorted, without a selection.
    const int64_t l = p.lens[row];
    const int64_t n_row = l < 0 ? 0 : (l < p.n ? l : p.n);
    if (n_row < static_cast<int64_t>(k)) {
      const uint32_t S = len / k;
      uint32_t at = 0;
      for (uint32_t s = 0; s < S; ++s) {
        const int64_t rest = n_row - static_cast<int64_t>(s) * p.slice_len;
        if (rest <= 0) break;  // slices are consecutive ranges: the rest are empty
        const uint32_t ls = static_cast<uint32_t>(rest < p.slice_len ? rest : p.slice_len);  // < k
        for (uint32_t i = tid; i < ls; i += NT) {
          const uint2 e = base[static_cast<uint64_t>(s) * k + i];
          L.ck[at + i] = e.x;
          L.ci[at + i] = e.y;
        }
        at += ls;
      }
      for (uint32_t i = at + tid; i < k; i += NT) {
        L.ck[i] = 0u;
        L.ci[i] = kSentinelIdx;
      }
      lds_sync();
      sort_and_store<DT, WAVES>(L.ck, L.ci, L.ck + L.k4, L.ci + L.k4, reinterpret_cast<uint64_t*>(L.hist), k,
                                p.out_vals, p.out_idx, nullptr, row);
      return;
    }
  }

  BlockOrder ord;
  ord.init(p.seed, row, 0x7FFFFFFFu, m);
  constexpr int D = depth_for(WAVES, CPW);
  FirstBlocks<D, CPW> fb;
  first_blocks<DT, WAVES, CPW, D, true>(rs, len, ord, 0u, fb);

  const OutSpec fso{p.out_vals, p.out_idx, nullptr, row};
  BodyOut bo;
  deepselect_body<DT, WAVES, CPW, D, true, false>(L, sc, rs, len, 0u, k, B2, ord, 0u, static_cast<uint32_t>(p.n - 1),
                                                  false, 0u, nullptr, p.presample != 0, 0u, fb, &fso, bo);
  if (bo.sorted) return;
  if (p.unsorted) {
    for (uint32_t i = tid; i < k; i += NT)
      store_out<DT>(p.out_vals, p.out_idx, nullptr, static_cast<uint64_t>(row) * k + i, comp_of(bo.fk[i], bo.fi[i]));
  } else {
    sort_and_store<DT, WAVES>(bo.fk, bo.fi, L.ck + L.k4, L.ci + L.k4, reinterpret_cast<uint64_t*>(L.hist), k,
                              p.out_vals, p.out_idx, nullptr, row);
  }
}

// --------------------------------------------------------------------------- list-merge kernel
// One level of the list merge: a row's p.lists sorted lists are merged in groups of p.group
// consecutive lists, each group into one sorted list of its k best (at p.dst, or the outputs
// when the level has one group). Each workgroup places p.per_wg lists of one group; the
// grid is rows x groups x ceil(group / per_wg), and workgroups past a short last group's
// lists return at once.
template <int DT, int WAVES, uint32_t MAXS, uint32_t EB>
//
// The parameters the first loads depend on come as scalars ahead of the rest (the grid's x
// size gx, groups gy and rows gz among them), preloaded into scalar registers at wave launch.
__global__ __launch_bounds__(WAVES * 64) void merge_lists_kernel(const uint2* pws, int64_t prow_entries, int64_t prow0,
                                                                 int32_t plists, int32_t pgroup, int32_t pper,
                                                                 int32_t pk_, int32_t ppk, int32_t gx, int32_t gy,
                                                                 int32_t gz, [[maybe_unused]] MergeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const uint32_t S = static_cast<uint32_t>(plists), G = static_cast<uint32_t>(pgroup);
  const uint32_t per = static_cast<uint32_t>(pper), k = static_cast<uint32_t>(pk_);
  // grid: (workgroups per group, groups, rows of this launch); a row's workgroups run on the
  // XCD that ran its slices (row0 is a multiple of 8), whose L2 holds their lists
  const uint32_t gxu = static_cast<uint32_t>(gx), wpr = gxu * static_cast<uint32_t>(gy);
  uint32_t lrow, r;
  xcd_unit(blockIdx.x + gxu * (blockIdx.y + static_cast<uint32_t>(gy) * blockIdx.z), wpr, static_cast<uint32_t>(gz),
           lrow, r);
  const uint64_t row = static_cast<uint64_t>(prow0) + lrow;
  uint32_t g, l0;
  divmod_uniform(r, gxu, g, l0);
  l0 *= per;
  const uint32_t first = g * G, gl = min(G, S - first);  // the group's lists
  if (l0 >= gl) return;  // the same for the whole workgroup
  const uint32_t pk = gl == G ? static_cast<uint32_t>(ppk) : (k + gl - 1u) / gl;  // ceil(k / gl)
  const uint2* src = pws + row * prow_entries + static_cast<uint64_t>(first) * k;
  // The output parameters come from the argument block in memory, read through a pointer
  // the compiler cannot hoist above the lists' loads (their waits would come first).
  auto outs = [&]() {
    const MergeParams& q = params_after_loads<MergeParams, kMergeParamsOffset>();
    MergeOut o;
    o.vals = q.out_vals;
    o.idx = IdxOut{q.out_idx.p, q.out_idx.wide};
    o.pairs = q.dst ? q.dst + row * q.dst_row_entries + static_cast<uint64_t>(g) * k : nullptr;
    o.at0 = q.dst ? 0u : row * k;
    return o;
  };
  merge_lists_t<DT, WAVES, MAXS, EB>(src, gl, k, pk, reinterpret_cast<uint64_t*>(lds), outs, l0, min(l0 + per, gl));
}

// Raises kernel KERN's dynamic-LDS limit to at least `lds` bytes on the current device. The
// attribute is set only when a larger size than before is asked for on that device, so the
// runtime call stays off the steady-state launch path.
constexpr int kAttrDevices = 64;
template <auto KERN>
hipError_t allow_lds(size_t lds) {
  static std::atomic<int> granted[kAttrDevices];  // zero-initialised: nothing granted yet
  if (lds <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kAttrDevices && granted[dev].load(std::memory_order_relaxed) >= static_cast<int>(lds))
    return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds));
  if (e == hipSuccess && dev >= 0 && dev < kAttrDevices) {
    int cur = granted[dev].load(std::memory_order_relaxed);
    while (cur < static_cast<int>(lds) && !granted[dev].compare_exchange_weak(cur, static_cast<int>(lds))) {
    }
  }
  return e;
}

}  // namespace
}  // namespace ds
