// A CPU model of the library's signal protocols, run under ThreadSanitizer.
//
// Test infrastructure: it shares no code with the kernels.  Threads play
// the workgroups; plain int32/int64 arrays play the data in HBM and
// std::atomic<int64_t> slots play the flags and counters, with the orderings
// the kernels use (a release before every publish or arrival, an acquire
// after every wait or completing arrival; "Triton-distributed Semantics",
// Signal-Based Synchronization and Token-Based Data Dependency).  The data
// itself moves with plain loads and stores, so that any consumer read which
// the protocol does not order after its producer's write is a data race
// ThreadSanitizer reports, whatever the timing.  Seeded random pauses shake
// the interleavings.
//
// Protocols (one per section of the input file, see main):
//  ag   AllGather -> GEMM: producers move flag units (or W pieces of a unit,
//       each arriving on the unit's monotone counter, the arrival completing
//       a multiple of W publishing: signal ADD then SET) in the producer
//       order the input gives; consumers take row tiles in the consumer order
//       the input gives (the library's host mirror of its device rule), wait
//       on every unit a K-batch of the tile needs, then read the gathered
//       rows.  Own row tiles read the own shard and never wait.  Several
//       epochs run on the same flags and counters, without a reset.
//  a2a  all-to-all dispatch: chunks of slice rows handed out by a ticket;
//       producers arrive once per run of chunks of one slice, consumers that
//       find their slice incomplete take chunks too and arrive per chunk; the
//       arrival that completes a slice publishes its flag; consumers wait on
//       every slice their rows come from.
//  rs   GEMM -> ReduceScatter: own tiles store the accumulator and publish an
//       own-tile flag; peer tiles store a partial and publish the out flag,
//       then run a reduce job that waits for the own tiles and the peers'
//       partials it covers and writes out = acc + sum of partials.
//
// Mutations (last argument), each a planted protocol bug that the test
// expects ThreadSanitizer to report: ag: skip_wait (a consumer does not wait
// for the last K-batch), publish_early (the flag is set before the copy),
// relaxed (flag store and load without release/acquire), add_no_release
// (pieces arrive with a relaxed add); a2a: arrive_early (a chunk arrives
// before it is copied); rs: no_own_wait (a reduce job does not wait for the
// own tiles).
//
// Exit status: 0 when every output equals its plain definition, 1 when one
// differs, 2 on a bad input (ThreadSanitizer itself exits with 66 on a race).
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <random>
#include <sstream>
#include <string>
#include <thread>
#include <vector>

namespace {

using Flag = std::atomic<int64_t>;
std::string g_mut;

bool mut(const char* m) { return g_mut == m; }

// A short seeded pause: nothing, a yield, or a sleep of a few microseconds.
struct Jitter {
  std::mt19937_64 rng;
  explicit Jitter(uint64_t seed) : rng(seed) {}
  void operator()() {
    const unsigned r = (unsigned)(rng() % 16);
    if (r < 10) return;
    if (r < 14) {
      std::this_thread::yield();
      return;
    }
    std::this_thread::sleep_for(std::chrono::microseconds(1 + rng() % 20));
  }
};

void spin_until(const Flag& f, int64_t v, std::memory_order mo) {
  while (f.load(mo) < v) std::this_thread::yield();
}

int fail(const char* what) {
  std::fprintf(stderr, "model: %s\n", what);
  return 1;
}

// ------------------------------------------------------------------ AG-GEMM

int run_ag(std::istream& in) {
  int R, rank, W, P, Cn, epochs;
  int64_t shard_m, K, N, unit_rows, panels, batch_cols, batches, tile_rows, tile_cols;
  uint64_t seed;
  in >> R >> rank >> shard_m >> K >> N >> unit_rows >> panels >> batch_cols >> batches >> tile_rows >> tile_cols >>
      W >> P >> Cn >> epochs >> seed;
  if (!in || R < 1 || W < 1 || P < 1 || Cn < 1 || epochs < 1) return 2;
  const int64_t M = R * shard_m, units = R * panels * batches;
  const int64_t row_tiles = (M + tile_rows - 1) / tile_rows, col_tiles = (N + tile_cols - 1) / tile_cols;
  std::vector<std::vector<int32_t>> order(epochs, std::vector<int32_t>(units)),
      corder(epochs, std::vector<int32_t>(row_tiles));
  for (int e = 0; e < epochs; ++e) {
    for (auto& v : order[e]) in >> v;
    for (auto& v : corder[e]) in >> v;
  }
  if (!in) return 2;
  std::mt19937_64 rng(seed);
  std::vector<int32_t> shards(M * K), b(K * N);
  for (auto& v : shards) v = (int32_t)(rng() % 9) - 4;
  for (auto& v : b) v = (int32_t)(rng() % 9) - 4;
  std::vector<int32_t> g(M * K);
  std::vector<int64_t> c(M * N);
  std::vector<Flag> flags(units), cnt(units);
  for (auto& f : flags) f.store(0);
  for (auto& f : cnt) f.store(0);
  const std::memory_order rel = mut("relaxed") ? std::memory_order_relaxed : std::memory_order_release;
  const std::memory_order acq = mut("relaxed") ? std::memory_order_relaxed : std::memory_order_acquire;

  for (int e = 0; e < epochs; ++e) {
    const int64_t epoch = e + 1;
    std::fill(g.begin(), g.end(), -1000000);
    std::fill(c.begin(), c.end(), 0);
    std::vector<std::thread> th;
    for (int w = 0; w < P; ++w)
      th.emplace_back([&, w] {
        Jitter jit(seed * 131 + epoch * 7 + w);
        for (int64_t i = w; i < units * W; i += P) {
          const int32_t u = order[e][i / W];
          if (u < 0 || u >= units) continue;
          const int piece = (int)(i % W);
          const int64_t bt = u % batches, sp = u / batches, p = sp % panels, s = sp / panels;
          const int64_t r0 = p * unit_rows, rows = std::min(unit_rows, shard_m - r0);
          const int64_t c0 = bt * batch_cols, cols = std::min(batch_cols, K - c0);
          const int64_t lo = r0 + rows * piece / W, hi = r0 + rows * (piece + 1) / W;
          Flag& f = flags[u];
          if (mut("publish_early") && W == 1) f.store(epoch, rel);
          jit();
          for (int64_t r = lo; r < hi; ++r)
            for (int64_t k = c0; k < c0 + cols; ++k) g[(s * shard_m + r) * K + k] = shards[(s * shard_m + r) * K + k];
          jit();
          if (W == 1) {
            if (!mut("publish_early")) f.store(epoch, rel);
          } else {
            const std::memory_order add = mut("add_no_release") ? std::memory_order_relaxed : std::memory_order_acq_rel;
            const int64_t old = cnt[u].fetch_add(1, add);
            if (old % W == W - 1) f.store(epoch, rel);
          }
        }
      });
    for (int ci = 0; ci < Cn; ++ci)
      th.emplace_back([&, ci] {
        Jitter jit(seed * 977 + epoch * 13 + ci);
        for (int64_t j = ci; j < row_tiles * col_tiles; j += Cn) {
          const int64_t rt = corder[e][j / col_tiles], nt = j % col_tiles;
          const int64_t m0 = rt * tile_rows, m1 = std::min(m0 + tile_rows, M);
          const int64_t n0 = nt * tile_cols, n1 = std::min(n0 + tile_cols, N);
          const bool own = m0 >= rank * shard_m && m1 <= (rank + 1) * shard_m;
          std::vector<int64_t> acc((m1 - m0) * (n1 - n0), 0);
          for (int64_t bt = 0; bt < batches; ++bt) {
            const int64_t k0 = bt * batch_cols, k1 = std::min(k0 + batch_cols, K);
            if (!own && !(mut("skip_wait") && bt == batches - 1)) {
              // every unit covering rows [m0, m1) in batch bt
              for (int64_t r = m0; r < m1;) {
                const int64_t s = r / shard_m, p = (r - s * shard_m) / unit_rows;
                spin_until(flags[(s * panels + p) * batches + bt], epoch, acq);
                r = std::min(s * shard_m + (p + 1) * unit_rows, (s + 1) * shard_m);
              }
            }
            jit();
            for (int64_t m = m0; m < m1; ++m)
              for (int64_t k = k0; k < k1; ++k) {
                const int32_t a = own ? shards[m * K + k] : g[m * K + k];
                for (int64_t n = n0; n < n1; ++n) acc[(m - m0) * (n1 - n0) + n - n0] += (int64_t)a * b[k * N + n];
              }
          }
          for (int64_t m = m0; m < m1; ++m)
            for (int64_t n = n0; n < n1; ++n) c[m * N + n] = acc[(m - m0) * (n1 - n0) + n - n0];
        }
      });
    for (auto& t : th) t.join();
    if (g != shards) return fail("ag: gathered differs from the concatenated shards");
    for (int64_t u = 0; u < units; ++u)
      if (flags[u].load() != epoch) return fail("ag: a flag does not hold the epoch");
    for (int64_t m = 0; m < M; ++m)
      for (int64_t n = 0; n < N; ++n) {
        int64_t ref = 0;
        for (int64_t k = 0; k < K; ++k) ref += (int64_t)shards[m * K + k] * b[k * N + n];
        if (c[m * N + n] != ref) return fail("ag: C differs from the product");
      }
  }
  return 0;
}

// ------------------------------------------------------------------ dispatch

int run_a2a(std::istream& in) {
  int R, rank, E, topk, P, Cn, chunk_rows, tile_rows;
  int64_t T, H, N;
  uint64_t seed;
  in >> R >> rank >> T >> H >> N >> topk >> E >> chunk_rows >> tile_rows >> P >> Cn >> seed;
  if (!in || R < 1 || E < 1 || topk < 1 || chunk_rows < 1 || P < 1 || Cn < 1) return 2;
  std::vector<std::vector<int32_t>> route(R, std::vector<int32_t>(T * topk));
  for (auto& r : route)
    for (auto& v : r) in >> v;
  if (!in) return 2;
  const int64_t cap = T * std::min(topk, E);
  std::mt19937_64 rng(seed);
  std::vector<int32_t> x(R * T * H), w(E * H * N);
  for (auto& v : x) v = (int32_t)(rng() % 9) - 4;
  for (auto& v : w) v = (int32_t)(rng() % 9) - 4;
  // Layout (the layout kernel's job, done up front): rows of slice s by
  // (local expert, token).
  std::vector<int32_t> src(R * cap, -1), expert(R * cap, -1);
  std::vector<int64_t> rows(R, 0);
  for (int s = 0; s < R; ++s)
    for (int e = 0; e < E; ++e)
      for (int64_t t = 0; t < T; ++t)
        for (int k = 0; k < topk; ++k)
          if (route[s][t * topk + k] == rank * E + e) {
            if (rows[s] >= cap) return 2;
            src[s * cap + rows[s]] = (int32_t)t;
            expert[s * cap + rows[s]] = e;
            ++rows[s];
          }
  // Chunks in slice order (own slice first), as the ticket hands them out.
  std::vector<int> chunk_slice;
  std::vector<int64_t> chunk_r0, need(R, 0);
  for (int pos = 0; pos < R; ++pos) {
    const int s = (rank + pos) % R;
    for (int64_t r = 0; r < rows[s]; r += chunk_rows) {
      chunk_slice.push_back(s);
      chunk_r0.push_back(r);
      ++need[s];
    }
  }
  const int64_t total = (int64_t)chunk_slice.size();
  std::vector<int32_t> recv(R * cap * H, -1000000);
  std::vector<int64_t> y(R * cap * N, 0);
  std::vector<Flag> flags(R), arrivals(R);
  for (auto& f : flags) f.store(0);
  for (auto& f : arrivals) f.store(0);
  Flag ticket{0};
  const int64_t epoch = 1;
  for (int s = 0; s < R; ++s)
    if (rows[s] == 0) flags[s].store(epoch, std::memory_order_release);
  auto copy_chunk = [&](int64_t ch) {
    const int s = chunk_slice[ch];
    const int64_t r1 = std::min(chunk_r0[ch] + chunk_rows, rows[s]);
    for (int64_t r = chunk_r0[ch]; r < r1; ++r)
      for (int64_t h = 0; h < H; ++h) recv[(s * cap + r) * H + h] = x[((int64_t)s * T + src[s * cap + r]) * H + h];
  };
  auto arrive = [&](int s, int64_t n) {
    const int64_t old = arrivals[s].fetch_add(n, std::memory_order_acq_rel);
    if (old + n == need[s]) flags[s].store(epoch, std::memory_order_release);
  };
  // Expert-major tiles: expert e's rows in slice order, cut into tile_rows.
  struct Tile {
    int e;
    std::vector<int64_t> rowid;  // s * cap + r
    int last_pos;
  };
  std::vector<Tile> tiles;
  for (int e = 0; e < E; ++e) {
    std::vector<int64_t> ids;
    std::vector<int> pos_of;
    for (int pos = 0; pos < R; ++pos) {
      const int s = (rank + pos) % R;
      for (int64_t r = 0; r < rows[s]; ++r)
        if (expert[s * cap + r] == e) {
          ids.push_back(s * cap + r);
          pos_of.push_back(pos);
        }
    }
    for (size_t i = 0; i < ids.size(); i += tile_rows) {
      Tile t{e, {}, 0};
      for (size_t q = i; q < std::min(ids.size(), i + tile_rows); ++q) {
        t.rowid.push_back(ids[q]);
        t.last_pos = pos_of[q];
      }
      tiles.push_back(std::move(t));
    }
  }
  std::vector<std::thread> th;
  for (int wv = 0; wv < P; ++wv)
    th.emplace_back([&, wv] {
      Jitter jit(seed * 31 + wv);
      int pend_s = -1;
      int64_t pend_n = 0;
      for (int64_t ch; (ch = ticket.fetch_add(1, std::memory_order_relaxed)) < total;) {
        const int s = chunk_slice[ch];
        if (pend_n && s != pend_s) {
          arrive(pend_s, pend_n);
          pend_n = 0;
        }
        if (mut("arrive_early")) arrive(s, 1);
        jit();
        copy_chunk(ch);
        if (!mut("arrive_early")) {
          pend_s = s;
          ++pend_n;
        }
      }
      if (pend_n) arrive(pend_s, pend_n);
    });
  for (int ci = 0; ci < Cn; ++ci)
    th.emplace_back([&, ci] {
      Jitter jit(seed * 57 + ci);
      int waited = -1;
      for (size_t j = ci; j < tiles.size(); j += Cn) {
        const Tile& t = tiles[j];
        while (waited < t.last_pos) {
          ++waited;
          const int s = (rank + waited) % R;
          // help copy while the slice is incomplete and chunks are left
          while (flags[s].load(std::memory_order_acquire) < epoch) {
            const int64_t ch = ticket.fetch_add(1, std::memory_order_relaxed);
            if (ch >= total) {
              spin_until(flags[s], epoch, std::memory_order_acquire);
              break;
            }
            if (mut("arrive_early")) arrive(chunk_slice[ch], 1);
            copy_chunk(ch);
            if (!mut("arrive_early")) arrive(chunk_slice[ch], 1);
          }
        }
        jit();
        for (int64_t id : t.rowid)
          for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t h = 0; h < H; ++h) acc += (int64_t)recv[id * H + h] * w[((int64_t)t.e * H + h) * N + n];
            y[id * N + n] = acc;
          }
      }
    });
  for (auto& t : th) t.join();
  for (int s = 0; s < R; ++s) {
    if (flags[s].load() != epoch) return fail("a2a: a slice flag is not set");
    for (int64_t r = 0; r < rows[s]; ++r)
      for (int64_t n = 0; n < N; ++n) {
        int64_t ref = 0;
        for (int64_t h = 0; h < H; ++h)
          ref += (int64_t)x[((int64_t)s * T + src[s * cap + r]) * H + h] * w[((int64_t)expert[s * cap + r] * H + h) * N + n];
        if (y[(s * cap + r) * N + n] != ref) return fail("a2a: y differs from the routed product");
      }
  }
  return 0;
}

// ------------------------------------------------------------------ GEMM-RS

int run_rs(std::istream& in) {
  int R, rank, Cn;
  int64_t bm, K, N, tile;
  uint64_t seed;
  in >> R >> rank >> bm >> K >> N >> tile >> Cn >> seed;
  if (!in || R < 2 || Cn < 1 || tile < 1) return 2;
  const int64_t M = R * bm, tr = (bm + tile - 1) / tile, tc = (N + tile - 1) / tile, tpb = tr * tc;
  std::mt19937_64 rng(seed);
  std::vector<int32_t> a(M * K), b(K * N);
  for (auto& v : a) v = (int32_t)(rng() % 9) - 4;
  for (auto& v : b) v = (int32_t)(rng() % 9) - 4;
  std::vector<std::vector<int64_t>> peer_in(R, std::vector<int64_t>(bm * N)), peer_out(R, std::vector<int64_t>(bm * N));
  for (auto& p : peer_in)
    for (auto& v : p) v = (int64_t)(rng() % 1001) - 500;
  std::vector<int64_t> out(bm * N, -1000000000);
  std::vector<Flag> own_flags(tpb), out_flags(R * tpb);
  for (auto& f : own_flags) f.store(0);
  for (auto& f : out_flags) f.store(0);
  const int64_t epoch = 1;
  const int64_t J = (R - 1) * tpb;  // reduce jobs, one per peer tile
  // own-row space: tile t owns rows [t*tile, (t+1)*tile); job j covers [j*OR/J, (j+1)*OR/J)
  const int64_t OR = tpb * tile;
  std::vector<std::thread> th;
  for (int ci = 0; ci < Cn; ++ci)
    th.emplace_back([&, ci] {
      Jitter jit(seed * 17 + ci);
      for (int64_t j = ci; j < R * tpb; j += Cn) {
        const int64_t pj = j - tpb;
        const int blk = pj < 0 ? rank : (int)((rank + 1 + pj / tpb) % R);
        const int64_t t = pj < 0 ? j : pj % tpb;
        const int64_t m0 = (t / tc) * tile, m1 = std::min(m0 + tile, bm);
        const int64_t n0 = (t % tc) * tile, n1 = std::min(n0 + tile, N);
        std::vector<int64_t> acc((m1 - m0) * (n1 - n0), 0);
        for (int64_t m = m0; m < m1; ++m)
          for (int64_t k = 0; k < K; ++k)
            for (int64_t n = n0; n < n1; ++n)
              acc[(m - m0) * (n1 - n0) + n - n0] += (int64_t)a[(blk * bm + m) * K + k] * b[k * N + n];
        jit();
        auto& dst = blk == rank ? out : peer_out[blk];
        for (int64_t m = m0; m < m1; ++m)
          for (int64_t n = n0; n < n1; ++n) dst[m * N + n] = acc[(m - m0) * (n1 - n0) + n - n0];
        if (blk == rank) {
          own_flags[t].store(epoch, std::memory_order_release);
          continue;
        }
        out_flags[blk * tpb + t].store(epoch, std::memory_order_release);
        // reduce job pj
        const int64_t q0 = pj * OR / J, q1 = (pj + 1) * OR / J;
        if (q0 >= q1) continue;
        if (!mut("no_own_wait"))
          for (int64_t tt = q0 / tile; tt <= (q1 - 1) / tile; ++tt) spin_until(own_flags[tt], epoch, std::memory_order_acquire);
        jit();
        for (int64_t q = q0; q < q1; ++q) {
          const int64_t tt = q / tile, row = (tt / tc) * tile + q % tile;
          if (row >= bm) continue;
          for (int64_t col = (tt % tc) * tile; col < std::min((tt % tc + 1) * tile, N); ++col) {
            int64_t sum = 0;
            for (int p = 0; p < R; ++p)
              if (p != rank) sum += peer_in[p][row * N + col];
            out[row * N + col] += sum;
          }
        }
      }
    });
  for (auto& t : th) t.join();
  for (int64_t m = 0; m < bm; ++m)
    for (int64_t n = 0; n < N; ++n) {
      int64_t ref = 0;
      for (int64_t k = 0; k < K; ++k) ref += (int64_t)a[(rank * bm + m) * K + k] * b[k * N + n];
      for (int p = 0; p < R; ++p)
        if (p != rank) ref += peer_in[p][m * N + n];
      if (out[m * N + n] != ref) return fail("rs: the own block differs from product + partials");
    }
  for (int p = 0; p < R; ++p) {
    if (p == rank) continue;
    for (int64_t t = 0; t < tpb; ++t)
      if (out_flags[p * tpb + t].load() != epoch) return fail("rs: an out flag is not set");
  }
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) {
    std::fprintf(stderr, "usage: %s INPUT [MUTATION]\n", argv[0]);
    return 2;
  }
  if (argc > 2) g_mut = argv[2];
  std::ifstream f(argv[1]);
  std::string kind;
  f >> kind;
  if (kind == "ag") return run_ag(f);
  if (kind == "a2a") return run_a2a(f);
  if (kind == "rs") return run_rs(f);
  return 2;
}
