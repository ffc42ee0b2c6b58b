// CPU oracle for row-wise top-k selection. TEST INFRASTRUCTURE ONLY.
//
// Only the tests, the smoke check and the benchmark's CPU-baseline leg may load this
// library. The product path never calls it and shares no code with it.
//
// What it computes (the plain definition of the result that DeepSelect reaches):
// for every row r, order the pairs (x[r][j], j), 0 <= j < N, by value descending and,
// among equal values, by index ascending (the smaller index wins a tie, the convention
// of the TileKernels top-k gate), then return the first k pairs. Values are returned as
// the input's own bit patterns, indices as int32 relative to the row.
//
// Sources: the DeepSelect design note ("Algorithm": RadixSelectTopK reduces the
// candidates to the k largest; the method is exact), the DeepSelect tutorial chapter
// (section 1.3: top-k of a row), and the TileKernels chapter (sections 2.1 and 4.1: a
// full stable sort as the "slow but correct" reference, ties to the smaller index).
//
// Readings taken where the pages are silent:
//  * +0 and -0 compare equal as numbers; this oracle ranks +0 before -0 (sign decides
//    between the two zeros, before the index does). All other ties go by index.
//  * NaN is outside the contract (the caller guarantees none).
//  * bf16 is widened to float by placing its 16 bits in the high half (exact), then to
//    double; every comparison is a numeric comparison of doubles.
//
// The order is implemented by an explicit comparator on numbers. It never uses an
// ordered-integer image of the floating-point bits.
//
// Parallelism: rows are spread over threads. A row longer than 2^20 elements with fewer
// rows than threads is fully sorted as per-thread chunks (each chunk a full std::sort)
// followed by a merge of the sorted chunks; the merge stops once the first k pairs of the
// merged order are out, which are by construction the first k of the full sorted row.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

struct Item {
  double v;       // numeric value, widened exactly
  uint32_t j;     // index in the row
  uint32_t bits;  // the input's bit pattern (16 or 32 bits)
};

// True when a ranks strictly before b in the output order.
inline bool ranks_before(const Item& a, const Item& b) {
  if (a.v > b.v) return true;
  if (a.v < b.v) return false;
  const bool a_neg = std::signbit(a.v), b_neg = std::signbit(b.v);
  if (a_neg != b_neg) return b_neg;  // only +0 / -0 reach here: +0 first
  return a.j < b.j;
}

inline Item load(const void* x, int dtype, int64_t off, uint32_t j) {
  Item it;
  it.j = j;
  if (dtype == 0) {
    uint16_t h;
    std::memcpy(&h, static_cast<const uint8_t*>(x) + off * 2, 2);
    uint32_t u = static_cast<uint32_t>(h) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    it.v = static_cast<double>(f);
    it.bits = h;
  } else {
    uint32_t u;
    std::memcpy(&u, static_cast<const uint8_t*>(x) + off * 4, 4);
    float f;
    std::memcpy(&f, &u, 4);
    it.v = static_cast<double>(f);
    it.bits = u;
  }
  return it;
}

void store(void* out_vals, int32_t* out_idx, int dtype, int64_t pos, const Item& it) {
  if (out_vals) {
    if (dtype == 0) {
      uint16_t h = static_cast<uint16_t>(it.bits);
      std::memcpy(static_cast<uint8_t*>(out_vals) + pos * 2, &h, 2);
    } else {
      std::memcpy(static_cast<uint8_t*>(out_vals) + pos * 4, &it.bits, 4);
    }
  }
  if (out_idx) out_idx[pos] = static_cast<int32_t>(it.j);
}

void row_serial(const void* x, int64_t n, int64_t row_off, int k, int dtype, void* out_vals, int32_t* out_idx,
                int64_t out_off) {
  std::vector<Item> items(static_cast<size_t>(n));
  for (int64_t j = 0; j < n; ++j) items[j] = load(x, dtype, row_off + j, static_cast<uint32_t>(j));
  std::sort(items.begin(), items.end(), ranks_before);
  for (int i = 0; i < k; ++i) store(out_vals, out_idx, dtype, out_off + i, items[i]);
}

void row_chunked(const void* x, int64_t n, int64_t row_off, int k, int dtype, void* out_vals, int32_t* out_idx,
                 int64_t out_off, int threads) {
  std::vector<Item> items(static_cast<size_t>(n));
  const int64_t chunk = (n + threads - 1) / threads;
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) {
    pool.emplace_back([&, t] {
      const int64_t lo = std::min<int64_t>(n, t * chunk), hi = std::min<int64_t>(n, lo + chunk);
      for (int64_t j = lo; j < hi; ++j) items[j] = load(x, dtype, row_off + j, static_cast<uint32_t>(j));
      std::sort(items.begin() + lo, items.begin() + hi, ranks_before);
    });
  }
  for (auto& th : pool) th.join();
  // merge the sorted chunks by repeatedly taking the best head
  std::vector<int64_t> head(threads), end(threads);
  for (int t = 0; t < threads; ++t) {
    head[t] = std::min<int64_t>(n, t * chunk);
    end[t] = std::min<int64_t>(n, head[t] + chunk);
  }
  for (int i = 0; i < k; ++i) {
    int best = -1;
    for (int t = 0; t < threads; ++t) {
      if (head[t] >= end[t]) continue;
      if (best < 0 || ranks_before(items[head[t]], items[head[best]])) best = t;
    }
    store(out_vals, out_idx, dtype, out_off + i, items[head[best]]);
    ++head[best];
  }
}

}  // namespace

extern "C" {

int oracle_hw_threads(void) {
  unsigned t = std::thread::hardware_concurrency();
  return t == 0 ? 1 : static_cast<int>(t);
}

// x: host pointer to rows*row_stride elements (dtype 0 = bf16 bits, 1 = fp32).
// out_vals: host [rows, k] of the input's element type, or NULL.
// out_idx:  host [rows, k] int32, or NULL.
// threads <= 0 means hardware_concurrency(). Returns 0, or -1 on invalid arguments.
int oracle_topk(const void* x, int64_t rows, int64_t n, int64_t row_stride, int k, int dtype, void* out_vals,
                int32_t* out_idx, int threads) {
  if (rows < 0 || n < 1 || row_stride < n || k < 1 || k > n || (dtype != 0 && dtype != 1)) return -1;
  if (n > INT32_MAX) return -1;
  if (rows == 0) return 0;
  if (!x || (!out_vals && !out_idx)) return -1;
  if (threads <= 0) threads = oracle_hw_threads();
  if (rows < threads && n >= (int64_t(1) << 20) && threads > 1) {
    for (int64_t r = 0; r < rows; ++r)
      row_chunked(x, n, r * row_stride, k, dtype, out_vals, out_idx, r * k, threads);
    return 0;
  }
  std::atomic<int64_t> next(0);
  const int nt = static_cast<int>(std::min<int64_t>(threads, rows));
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    pool.emplace_back([&] {
      for (int64_t r = next++; r < rows; r = next++)
        row_serial(x, n, r * row_stride, k, dtype, out_vals, out_idx, r * k);
    });
  }
  for (auto& th : pool) th.join();
  return 0;
}

}  // extern "C"
