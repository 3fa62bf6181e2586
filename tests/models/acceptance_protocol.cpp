// CPU model of the single-read acceptance protocol (the cross-workgroup
// exchange of the acceptance kernel), run with one thread per resident
// workgroup slot.
//
// What is modelled, step for step as the kernel takes them:
//   * items (row, chunk) are dispatched in increasing order onto at most
//     `resident` slots at a time (a slot frees when its item returns), as the
//     hardware dispatches workgroups of one grid;
//   * an item publishes its chunk pair of each row (max, sum) into a 64-bit
//     word that is never 0 once written, polls the row's words at most
//     `spin_limit` times, and otherwise computes every pair of the row itself
//     (same arithmetic, so the same bits) and re-publishes its own words with
//     an exchange;
//   * it folds the row normalisers, sums min(p, q) over its chunk and arrives
//     on the row's word with (1 << 53) + the fixed-point sum; the arrival that
//     finds count == chunks - 1 writes alpha and clears the row's pair words
//     and its own word.
// The arithmetic inside a chunk is simplified (one max and sum per chunk
// instead of per thread): the protocol, not the rounding, is modelled.
// Checked over many seeded trials: every call returns (no item waits
// without bound), alpha equals a single-threaded evaluation of the same
// arithmetic bit for bit whatever the residency and spin limit, the sync
// region is all zero after every call (also across calls of different shapes
// on one workspace, and when fewer slots are resident than a row has chunks),
// and the fallback count is 0 when every item is resident with a generous
// limit.
//
// Memory order: the model uses release/acquire on the arrival and on pair
// reads to stand for the ordering the kernel obtains by completion (its pair
// reads feed the value it arrives with, and its own pair words were observed
// or exchanged before it arrives).
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

namespace {

constexpr int kCountShift = 53;
constexpr int kFixBits = 48;
constexpr int kWaves = 1;  // arrivals per item

struct Shape {
  int rows, vocab, chunk;
  int nchunk() const { return (vocab + chunk - 1) / chunk; }
};

uint64_t pack(float m, float s) {
  uint32_t a, b;
  std::memcpy(&a, &m, 4);
  std::memcpy(&b, &s, 4);
  return ((uint64_t)a << 32) | b;
}
float hi(uint64_t w) { uint32_t a = (uint32_t)(w >> 32); float f; std::memcpy(&f, &a, 4); return f; }
float lo(uint64_t w) { uint32_t a = (uint32_t)w; float f; std::memcpy(&f, &a, 4); return f; }

// Chunk pair of one row: max, then sum of 2^(x - max), entries in order.
void chunk_pair(const float* x, int n, float& m, float& s) {
  m = -INFINITY;
  for (int i = 0; i < n; ++i) m = std::fmax(m, x[i]);
  s = 0.f;
  for (int i = 0; i < n; ++i) s += std::exp2(x[i] - m);
}

struct Call {
  Shape sh;
  const std::vector<float>* a;
  const std::vector<float>* b;
  std::atomic<uint64_t>* pairs;  // [rows][2][nchunk]
  std::atomic<uint64_t>* word;   // [rows]
  std::vector<float>* alpha;
  int spin_limit;
  std::atomic<int>* fallbacks;
  std::mt19937* rng;
  std::mutex* rng_mu;
};

void jitter(const Call& c) {
  int d;
  {
    std::lock_guard<std::mutex> g(*c.rng_mu);
    d = (int)((*c.rng)() % 4);
  }
  if (d == 0) std::this_thread::yield();
  if (d == 1) std::this_thread::sleep_for(std::chrono::microseconds(1 + (d * 7) % 20));
}

void chunk_range(const Shape& sh, int ch, int& lo_i, int& n) {
  lo_i = ch * sh.chunk;
  n = std::min(sh.chunk, sh.vocab - lo_i);
}

void item(const Call& c, int it) {
  const Shape& sh = c.sh;
  const int S = sh.nchunk();
  const int r = it / S, ch = it % S;
  int i0, n;
  chunk_range(sh, ch, i0, n);
  const float* ra = c.a->data() + (size_t)r * sh.vocab;
  const float* rb = c.b->data() + (size_t)r * sh.vocab;
  float ma, sa, mb, sb;
  chunk_pair(ra + i0, n, ma, sa);
  chunk_pair(rb + i0, n, mb, sb);
  std::atomic<uint64_t>* rp = c.pairs + (size_t)r * 2 * S;
  jitter(c);
  rp[ch].store(pack(ma, sa), std::memory_order_relaxed);
  rp[S + ch].store(pack(mb, sb), std::memory_order_relaxed);
  std::vector<uint64_t> w(2 * S, 0);
  bool ready = false;
  for (int iter = 0;; ++iter) {
    bool all = true;
    for (int k = 0; k < 2 * S; ++k) {
      if (w[k] == 0) w[k] = rp[k].load(std::memory_order_acquire);
      all = all && w[k] != 0;
    }
    if (all) { ready = true; break; }
    if (iter >= c.spin_limit) break;
    std::this_thread::yield();
  }
  if (!ready) {
    for (int j = 0; j < S; ++j) {
      int j0, m;
      chunk_range(sh, j, j0, m);
      float x, y;
      chunk_pair(ra + j0, m, x, y);
      w[j] = pack(x, y);
      chunk_pair(rb + j0, m, x, y);
      w[S + j] = pack(x, y);
    }
    rp[ch].exchange(pack(ma, sa), std::memory_order_acq_rel);
    rp[S + ch].exchange(pack(mb, sb), std::memory_order_acq_rel);
    c.fallbacks->fetch_add(1);
  }
  float nrm[4];
  for (int row = 0; row < 2; ++row) {
    float M = -1e30f;
    for (int j = 0; j < S; ++j) M = std::fmax(M, hi(w[row * S + j]));
    float Z = 0.f;
    for (int j = 0; j < S; ++j) Z = std::fma(std::exp2(hi(w[row * S + j]) - M), lo(w[row * S + j]), Z);
    nrm[2 * row] = M;
    nrm[2 * row + 1] = 1.f / Z;
  }
  const float ka = std::exp2(ma - nrm[0]) * nrm[1], kb = std::exp2(mb - nrm[2]) * nrm[3];
  // each of the item's kWaves waves arrives with the sum over its share of the chunk
  for (int wv = 0; wv < kWaves; ++wv) {
    float cs = 0.f;
    for (int i = wv; i < n; i += kWaves)
      cs += std::fmin(std::exp2(ra[i0 + i] - ma) * ka, std::exp2(rb[i0 + i] - mb) * kb);
    const uint64_t fx = (uint64_t)std::llrint((double)cs * (double)(1ull << kFixBits));
    jitter(c);
    const uint64_t old = c.word[r].fetch_add((1ull << kCountShift) + fx, std::memory_order_acq_rel);
    if ((int)(old >> kCountShift) == kWaves * S - 1) {
      const uint64_t tot = (old & ((1ull << kCountShift) - 1)) + fx;
      const float s = (float)((double)tot / (double)(1ull << kFixBits));
      (*c.alpha)[r] = std::fmin(1.f, std::fmax(0.f, s));
      c.word[r].store(0, std::memory_order_relaxed);
      for (int k = 0; k < 2 * S; ++k) rp[k].store(0, std::memory_order_relaxed);
    }
  }
}

// Single-threaded evaluation of the same arithmetic.
std::vector<float> reference(const Shape& sh, const std::vector<float>& a, const std::vector<float>& b) {
  const int S = sh.nchunk();
  std::vector<float> out(sh.rows);
  for (int r = 0; r < sh.rows; ++r) {
    std::vector<uint64_t> w(2 * S);
    for (int j = 0; j < S; ++j) {
      int j0, m;
      chunk_range(sh, j, j0, m);
      float x, y;
      chunk_pair(a.data() + (size_t)r * sh.vocab + j0, m, x, y);
      w[j] = pack(x, y);
      chunk_pair(b.data() + (size_t)r * sh.vocab + j0, m, x, y);
      w[S + j] = pack(x, y);
    }
    float nrm[4];
    for (int row = 0; row < 2; ++row) {
      float M = -1e30f;
      for (int j = 0; j < S; ++j) M = std::fmax(M, hi(w[row * S + j]));
      float Z = 0.f;
      for (int j = 0; j < S; ++j) Z = std::fma(std::exp2(hi(w[row * S + j]) - M), lo(w[row * S + j]), Z);
      nrm[2 * row] = M;
      nrm[2 * row + 1] = 1.f / Z;
    }
    uint64_t tot = 0;
    for (int j = 0; j < S; ++j) {
      int j0, m;
      chunk_range(sh, j, j0, m);
      const float* ra = a.data() + (size_t)r * sh.vocab + j0;
      const float* rb = b.data() + (size_t)r * sh.vocab + j0;
      const float ma = hi(w[j]), mb = hi(w[S + j]);
      const float ka = std::exp2(ma - nrm[0]) * nrm[1], kb = std::exp2(mb - nrm[2]) * nrm[3];
      for (int wv = 0; wv < kWaves; ++wv) {
        float cs = 0.f;
        for (int i = wv; i < m; i += kWaves)
          cs += std::fmin(std::exp2(ra[i] - ma) * ka, std::exp2(rb[i] - mb) * kb);
        tot += (uint64_t)std::llrint((double)cs * (double)(1ull << kFixBits));
      }
    }
    const float s = (float)((double)tot / (double)(1ull << kFixBits));
    out[r] = std::fmin(1.f, std::fmax(0.f, s));
  }
  return out;
}

// Runs one call: items dispatched in order onto `resident` slots.
int run_call(Call& c, int resident) {
  const int items = c.sh.rows * c.sh.nchunk();
  std::atomic<int> next{0};
  std::vector<std::thread> slots;
  for (int s = 0; s < std::min(resident, items); ++s)
    slots.emplace_back([&] {
      for (;;) {
        const int it = next.fetch_add(1);
        if (it >= items) return;
        item(c, it);
      }
    });
  for (auto& t : slots) t.join();
  return c.fallbacks->load();
}

}  // namespace

int main() {
  const size_t kSync = 4096;  // words of the modelled sync region
  std::vector<std::atomic<uint64_t>> sync(kSync);
  for (auto& x : sync) x.store(0);
  std::mt19937 rng(12345);
  std::mutex rng_mu;
  int failures = 0, calls = 0;
  const Shape shapes[] = {{1, 4, 8}, {3, 37, 8}, {5, 100, 16}, {8, 256, 32}, {4, 1000, 64}, {16, 320, 20}, {2, 7, 7}};
  for (int trial = 0; trial < 400; ++trial) {
    const Shape sh = shapes[trial % (sizeof(shapes) / sizeof(shapes[0]))];
    const int S = sh.nchunk(), items = sh.rows * S;
    std::normal_distribution<float> nd(0.f, 3.f);
    std::vector<float> a((size_t)sh.rows * sh.vocab), b(a.size());
    for (size_t i = 0; i < a.size(); ++i) {
      a[i] = nd(rng);
      b[i] = a[i] + 0.1f * nd(rng);
    }
    std::vector<float> alpha(sh.rows, -1.f);
    std::atomic<int> fb{0};
    Call c{sh, &a, &b, sync.data(), sync.data() + 2 * items + 64, &alpha, 0, &fb, &rng, &rng_mu};
    // resident slots: all items, fewer than a row's chunks, or in between
    const int mode = trial % 4;
    const int resident = mode == 0 ? items : mode == 1 ? std::max(1, S - 1) : std::max(1, items / 2);
    c.spin_limit = mode == 3 ? 0 : (mode == 1 ? 50 : 200000);
    const int nfb = run_call(c, mode == 3 ? items : resident);
    ++calls;
    const std::vector<float> want = reference(sh, a, b);
    bool ok = std::memcmp(want.data(), alpha.data(), sizeof(float) * sh.rows) == 0;
    for (size_t i = 0; i < kSync; ++i) ok = ok && sync[i].load() == 0;
    if (mode == 0 && nfb != 0) ok = false;   // all resident, generous limit: nobody stops waiting
    if (nfb > items) ok = false;
    if (!ok) {
      ++failures;
      std::printf("FAIL trial %d rows %d vocab %d chunk %d resident %d limit %d fallbacks %d\n", trial, sh.rows,
                  sh.vocab, sh.chunk, resident, c.spin_limit, nfb);
    }
  }
  std::printf("%d calls, %d failures\n", calls, failures);
  return failures == 0 ? 0 : 1;
}
