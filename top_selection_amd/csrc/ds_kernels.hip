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

__device__ __forceinline__ uint32_t shfl(uint32_t v, uint32_t src_lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(static_cast<int>(src_lane << 2), static_cast<int>(v)));
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t o = 32; o > 0; o >>= 1) v |= shfl(v, lane ^ o);
  return v;
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v, uint32_t lane) {
#pragma unroll
  for (uint32_t o = 32; o > 0; o >>= 1) v &= shfl(v, lane ^ o);
  return v;
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

struct Scalars {
  uint32_t app_count;              // entries appended since the last compaction
  uint32_t outpos;                 // scatter cursor of the running compaction
  uint32_t slot[2][kMaxWaves];     // per-wave end of its reservation, by block parity
  uint32_t red[kMaxWaves][4];      // OR/AND reductions of the compaction
  uint32_t mred[kMaxWaves][2];     // min-composite reduction of the compaction
  unsigned long long reads;        // counters (stats runs only)
  unsigned long long index_sum;
};

struct Thr {
  uint32_t key, idx;
};

// Every wave scans the same 256-bin histogram (bins in descending digit order) and finds the
// bin holding the `need`-th best entry: `above` entries lie in higher bins, `cnt` in it.
__device__ __forceinline__ void scan_select(const uint32_t* h, uint32_t need, uint32_t lane, uint32_t& bin,
                                            uint32_t& above, uint32_t& cnt) {
  const uint32_t top = 255u - 4u * lane;  // this lane holds bins top, top-1, top-2, top-3
  const uint4 q = *reinterpret_cast<const uint4*>(h + top - 3);
  const uint32_t c0 = q.w, c1 = q.z, c2 = q.y, c3 = q.x;
  const uint32_t s = c0 + c1 + c2 + c3;
  uint32_t incl = s;
#pragma unroll
  for (uint32_t d = 1; d < 64; d <<= 1) {
    const uint32_t t = shfl(incl, lane >= d ? lane - d : lane);
    if (lane >= d) incl += t;
  }
  const uint64_t ge = ballot(incl >= need);
  const uint32_t src = ge ? static_cast<uint32_t>(__builtin_ctzll(ge)) : 63u;
  const uint32_t excl = incl - s;
  uint32_t b, a, c;
  if (excl + c0 >= need) {
    b = top; a = excl; c = c0;
  } else if (excl + c0 + c1 >= need) {
    b = top - 1; a = excl + c0; c = c1;
  } else if (excl + c0 + c1 + c2 >= need) {
    b = top - 2; a = excl + c0 + c1; c = c2;
  } else {
    b = top - 3; a = excl + c0 + c1 + c2; c = c3;
  }
  bin = __builtin_amdgcn_readlane(b, src);
  above = __builtin_amdgcn_readlane(a, src);
  cnt = __builtin_amdgcn_readlane(c, src);
}

// Radix-select compaction: reduce the nsurv survivors in `sin` plus the napp appended entries
// in `app` to the k best under the composite order, written (unordered) to `sout`, and
// return the smallest of them (the new threshold). When the input holds at most k entries
// everything is kept and `sout` is padded with sentinels up to k. RAW: appended entries hold
// raw element bits (bf16: in the high half) and are turned into keys here.
template <int DT, int WAVES, bool RAW>
__device__ Thr compact(const uint2* sin, uint32_t nsurv, uint2* app, uint32_t napp, uint2* sout, uint32_t k,
                       Scalars& sc, uint32_t* hist3, uint32_t& hctr) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t n = nsurv + napp;

  // 1. keys for the new entries; OR / AND of keys and of inverted indices over the buffer
  uint32_t ok = 0, ak = ~0u, oi = 0, ai = ~0u;
  for (uint32_t i = tid; i < n; i += NT) {
    uint2 e;
    if (i < nsurv) {
      e = sin[i];
    } else {
      e = app[i - nsurv];
      if constexpr (RAW) {
        e.x = key_of_raw<DT>(DT == DS_BF16 ? (e.x >> 16) : e.x);
        app[i - nsurv].x = e.x;
      }
    }
    ok |= e.x;
    ak &= e.x;
    oi |= ~e.y;
    ai &= ~e.y;
  }
  ok = wave_or(ok, lane);
  ak = wave_and(ak, lane);
  oi = wave_or(oi, lane);
  ai = wave_and(ai, lane);
  if (lane == 0) {
    sc.red[wave][0] = ok;
    sc.red[wave][1] = ak;
    sc.red[wave][2] = oi;
    sc.red[wave][3] = ai;
  }
  if (tid == 0) {
    sc.outpos = 0;
    sc.app_count = 0;
  }
  lds_sync();
  ok = 0;
  ak = ~0u;
  oi = 0;
  ai = ~0u;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    ok |= sc.red[w][0];
    ak &= sc.red[w][1];
    oi |= sc.red[w][2];
    ai &= sc.red[w][3];
  }

  // 2. radix select of the k-th best composite: first over key bits, then over ~index bits
  const bool all = n <= k;
  uint32_t need = k, pk = 0, pi = 0;
  if (!all) {
    bool done = false;
    const uint32_t dk = ok ^ ak;
    if (dk == 0) {
      pk = ak;  // every key equal: only the index decides
    } else {
      int hb = 31 - __builtin_clz(dk);
      uint32_t mk = hb == 31 ? 0u : (~0u << (hb + 1));
      pk = ak & mk;
      int lo = hb > 7 ? hb - 7 : 0;
      for (;;) {
        const uint32_t dmask = (1u << (hb - lo + 1)) - 1u;
        uint32_t* h = hist3 + 256u * (hctr % 3u);
        uint32_t* hn = hist3 + 256u * ((hctr + 1u) % 3u);
        for (uint32_t b = tid; b < 256u; b += NT) hn[b] = 0;
        for (uint32_t i = tid; i < n; i += NT) {
          const uint32_t key = (i < nsurv ? sin[i] : app[i - nsurv]).x;
          if ((key & mk) == pk) atomicAdd(&h[(key >> lo) & dmask], 1u);
        }
        lds_sync();
        ++hctr;
        uint32_t bin, above, cnt;
        scan_select(h, need, lane, bin, above, cnt);
        need -= above;
        pk |= bin << lo;
        mk |= dmask << lo;
        if (cnt == need) {
          done = true;
          break;
        }
        if (lo == 0) break;
        hb = lo - 1;
        lo = hb > 7 ? hb - 7 : 0;
      }
    }
    if (!done) {
      // `need` more entries among those whose key equals pk: the smallest indices win
      const uint32_t di = oi ^ ai;
      int hb = di ? 31 - __builtin_clz(di) : 0;
      uint32_t mi = hb == 31 ? 0u : (~0u << (hb + 1));
      pi = ai & mi;
      int lo = hb > 7 ? hb - 7 : 0;
      for (;;) {
        const uint32_t dmask = (1u << (hb - lo + 1)) - 1u;
        uint32_t* h = hist3 + 256u * (hctr % 3u);
        uint32_t* hn = hist3 + 256u * ((hctr + 1u) % 3u);
        for (uint32_t b = tid; b < 256u; b += NT) hn[b] = 0;
        for (uint32_t i = tid; i < n; i += NT) {
          const uint2 e = i < nsurv ? sin[i] : app[i - nsurv];
          const uint32_t ni = ~e.y;
          if (e.x == pk && (ni & mi) == pi) atomicAdd(&h[(ni >> lo) & dmask], 1u);
        }
        lds_sync();
        ++hctr;
        uint32_t bin, above, cnt;
        scan_select(h, need, lane, bin, above, cnt);
        need -= above;
        pi |= bin << lo;
        mi |= dmask << lo;
        if (cnt == need || lo == 0) break;
        hb = lo - 1;
        lo = hb > 7 ? hb - 7 : 0;
      }
    }
  }

  // 3. scatter the selected entries (composite >= (pk, pi)) and find the smallest of them
  uint32_t min_key = ~0u, min_ni = ~0u;
  const uint32_t iters = (n + NT - 1) / NT;
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t i = it * NT + tid;
    bool sel = false;
    uint2 e = make_uint2(0, 0);
    if (i < n) {
      e = i < nsurv ? sin[i] : app[i - nsurv];
      sel = all || e.x > pk || (e.x == pk && ~e.y >= pi);
    }
    const uint64_t bm = ballot(sel);
    if (bm) {
      uint32_t b0 = 0;
      if (lane == 0) b0 = atomicAdd(&sc.outpos, popc(bm));
      b0 = uni(b0);
      if (sel) {
        sout[mbcnt(bm, b0)] = e;
        if (e.x < min_key || (e.x == min_key && ~e.y < min_ni)) {
          min_key = e.x;
          min_ni = ~e.y;
        }
      }
    }
  }
  if (all) {
    for (uint32_t i = n + tid; i < k; i += NT) sout[i] = make_uint2(0, kSentinelIdx);
  }
#pragma unroll
  for (uint32_t o = 32; o > 0; o >>= 1) {
    const uint32_t ok2 = shfl(min_key, lane ^ o), on2 = shfl(min_ni, lane ^ o);
    if (ok2 < min_key || (ok2 == min_key && on2 < min_ni)) {
      min_key = ok2;
      min_ni = on2;
    }
  }
  if (lane == 0) {
    sc.mred[wave][0] = min_key;
    sc.mred[wave][1] = min_ni;
  }
  lds_sync();
  min_key = ~0u;
  min_ni = ~0u;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const uint32_t a = sc.mred[w][0], b = sc.mred[w][1];
    if (a < min_key || (a == min_key && b < min_ni)) {
      min_key = a;
      min_ni = b;
    }
  }
  return Thr{min_key, ~min_ni};
}

// Bitonic sort of cap (a power of two) entries, best first, then store the first k.
template <int DT, int WAVES>
__device__ void sort_and_store(uint2* sb, const uint2* fin, uint32_t k, uint32_t cap, void* out_vals,
                               int32_t* out_idx, uint64_t row) {
  constexpr uint32_t NT = WAVES * 64;
  const uint32_t tid = threadIdx.x;
  for (uint32_t i = tid; i < cap; i += NT) sb[i] = i < k ? fin[i] : make_uint2(0, kSentinelIdx);
  lds_sync();
  for (uint32_t size = 2; size <= cap; size <<= 1) {
    for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (uint32_t q = tid; q < cap / 2; q += NT) {
        const uint32_t i = ((q & ~(stride - 1)) << 1) | (q & (stride - 1));
        const uint32_t j = i + stride;
        const uint2 a = sb[i], b = sb[j];
        const bool desc = (i & size) == 0;
        const bool b_first = b.x > a.x || (b.x == a.x && b.y < a.y);
        if (b_first == desc) {
          sb[i] = b;
          sb[j] = a;
        }
      }
      lds_sync();
    }
  }
  for (uint32_t i = tid; i < k; i += NT) {
    const uint2 e = sb[i];
    if (out_vals) {
      if constexpr (DT == DS_BF16)
        static_cast<uint16_t*>(out_vals)[row * k + i] = static_cast<uint16_t>(raw_of_key<DT>(e.x));
      else
        static_cast<uint32_t*>(out_vals)[row * k + i] = raw_of_key<DT>(e.x);
    }
    if (out_idx) out_idx[row * k + i] = static_cast<int32_t>(e.y);
  }
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

  for (uint32_t i = tid; i < 768u; i += NT) hist3[i] = 0;
  if (tid == 0) {
    sc.app_count = 0;
    sc.outpos = 0;
    sc.reads = 0;
    sc.index_sum = 0;
  }

  const uint8_t* base = p.x + static_cast<uint64_t>(row) * p.row_stride_bytes + static_cast<uint64_t>(slice_lo) * EB;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, static_cast<int>(len * EB), kRsrcWord3);
  BlockOrder ord;
  ord.init(p.seed, row, slice, m);

  // threshold state (uniform across the workgroup)
  uint32_t mode = 0, thr_s = 0, thr_n = 0, t_idx = 0;
  Thr prev_t{0, kSentinelIdx};
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
        const Thr t = compact<DT, WAVES, true>(sin, nsurv, nsurv ? app_main : app_warm, napp, sout, k, sc, hist3,
                                               hctr);
        st_a += napp;
        st_w += nsurv + napp;
        st_r += 1;
        if (t.key < prev_t.key || (t.key == prev_t.key && t.idx > prev_t.idx)) st_mono = 0;
        prev_t = t;
        cur = nsurv ? (cur ^ 1u) : 0u;
        nsurv = k;
        napp = 0;
        t_idx = t.idx;
        filter_thresholds<DT>(t, mode, thr_s, thr_n);
      }
    }
  }

  // ---- final compaction
  uint2* const fin = nsurv ? (cur ? surv0 : surv1) : surv0;
  {
    const uint2* const sin = cur ? surv1 : surv0;
    compact<DT, WAVES, true>(sin, nsurv, nsurv ? app_main : app_warm, napp, fin, k, sc, hist3, hctr);
    st_a += napp;
    st_w += nsurv + napp;
  }

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
    sort_and_store<DT, WAVES>(app_main, fin, k, static_cast<uint32_t>(p.sort_cap), p.out_vals, p.out_idx, row);
  } else {
    uint2* const dst = p.ws + static_cast<uint64_t>(blockIdx.x) * k;
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

  for (uint32_t i = tid; i < 768u; i += NT) hist3[i] = 0;
  if (tid == 0) {
    sc.app_count = 0;
    sc.outpos = 0;
  }
  const uint2* base = p.ws + static_cast<uint64_t>(row) * len;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint2*>(base), 0, static_cast<int>(len * 8u), kRsrcWord3);
  BlockOrder ord;
  ord.init(p.seed, row, 0x7FFFFFFFu, m);

  bool accept_all = true;
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
        thr = compact<DT, WAVES, false>(sin, nsurv, nsurv ? app_main : app_warm, napp, sout, k, sc, hist3, hctr);
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
    compact<DT, WAVES, false>(sin, nsurv, nsurv ? app_main : app_warm, napp, fin, k, sc, hist3, hctr);
  }
  sort_and_store<DT, WAVES>(app_main, fin, k, static_cast<uint32_t>(p.sort_cap), p.out_vals, p.out_idx, row);
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
  return (static_cast<size_t>(2) * k + slack + block + 1) * 8 + 768 * 4 + sizeof(Scalars);
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
