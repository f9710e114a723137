// Host-side validation and scheduling (no HIP dependency).
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cmath>
#include <cstdio>
#include <numeric>
#include <queue>
#include <sstream>

namespace muon {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

std::string fmt(const char *f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

}  // namespace

size_t dtype_size(int32_t dtype) {
  switch (dtype) {
    case MUON_F32: return 4;
    case MUON_BF16: return 2;
    default: return 0;
  }
}

Layout view_layout(int64_t mp, int64_t np, bool bf16, bool distributed) {
  const size_t es = bf16 ? 2 : 4;
  const size_t mn = size_t(mp) * size_t(np) * es;
  const size_t mm = size_t(mp) * size_t(mp) * es;
  Layout L{};
  size_t off = 0;
  for (int p = 0; p < 2; ++p) {
    L.xa[p] = off;
    off = align_up(off + mn, 256);
  }
  for (int p = 0; p < 2; ++p) {
    L.xt[p] = off;
    if (bf16) off = align_up(off + mn, 256);
  }
  L.ahi = off;
  off = align_up(off + mm, 256);
  L.alo = off;
  if (bf16) off = align_up(off + mm, 256);
  L.b = off;
  off = align_up(off + mm, 256);
  L.bdiag = off;
  if (bf16) off = align_up(off + size_t(mp) * sizeof(float), 256);
  L.nparts = (mp / kElemTile) * (np / kElemTile);
  L.partials = off;
  off = align_up(off + size_t(L.nparts) * sizeof(float), 256);
  L.scale = off;
  off = align_up(off + 4 * sizeof(float), 256);
  L.tri = off;
  if (distributed) {
    // the shard's partial Gram as sent: bf16 path tile-packed (the upper
    // 256 x 256 tiles in float32), float32 path packed rows
    const size_t t = size_t(mp) / 256;
    off = align_up(off + (bf16 ? t * (t + 1) / 2 * 65536 : size_t(mp) * size_t(mp + 1) / 2) * sizeof(float), 256);
  }
  L.total = off;
  return L;
}

bool validate_mode(uint32_t mode, Error *err) {
  const uint32_t known = MUON_NS_BLOCKWISE | MUON_NS_DISTRIBUTED | MUON_PACK_COST | MUON_AA_SPLIT;
  if (mode & ~known) return err->set(MUON_ERR_INVALID_ARG, fmt("unknown mode bits 0x%llx", mode & ~known));
  if ((mode & MUON_NS_BLOCKWISE) && (mode & MUON_NS_DISTRIBUTED))
    return err->set(MUON_ERR_INVALID_ARG, "MUON_NS_BLOCKWISE and MUON_NS_DISTRIBUTED exclude each other");
  return true;
}

bool validate_descs(const muon_mat *d, int32_t n, uint32_t mode, const char *what, Error *err) {
  if (n < 0 || n > kMaxMats) return err->set(MUON_ERR_INVALID_ARG, fmt("n_mats %lld out of range", n));
  if (n > 0 && !d) return err->set(MUON_ERR_INVALID_ARG, std::string(what) + " is NULL");
  const bool blockwise = mode & MUON_NS_BLOCKWISE;
  const bool distributed = mode & MUON_NS_DISTRIBUTED;
  for (int32_t i = 0; i < n; ++i) {
    const muon_mat &x = d[i];
    const std::string who = std::string(what) + fmt("[%lld]", i);
    const size_t es = dtype_size(x.dtype);
    if (!es) return err->set(MUON_ERR_DTYPE, who + fmt(": unknown dtype %lld", x.dtype));
    if (x.dtype != d[0].dtype) return err->set(MUON_ERR_DTYPE, who + ": all matrices of a call must share one dtype");
    if (!x.data) return err->set(MUON_ERR_INVALID_ARG, who + ": data is NULL");
    if (x.rows <= 0 || x.cols <= 0) return err->set(MUON_ERR_SHAPE, who + fmt(": rows %lld, cols %lld must be positive", x.rows, x.cols));
    if (x.ld < x.cols) return err->set(MUON_ERR_SHAPE, who + fmt(": ld %lld < cols %lld", x.ld, x.cols));
    if (x.col_blocks < 0) return err->set(MUON_ERR_SHAPE, who + ": col_blocks < 0");
    int64_t k = ((blockwise || distributed) && x.col_blocks > 1) ? x.col_blocks : 1;
    if (x.cols % k) return err->set(MUON_ERR_SHAPE, who + fmt(": col_blocks %lld does not divide cols %lld", k, x.cols));
    if (distributed && std::max<int32_t>(x.col_blocks, 1) != std::max<int32_t>(d[0].col_blocks, 1))
      return err->set(MUON_ERR_SHAPE, who + ": distributed mode needs the same col_blocks (shard count) for every matrix");
    if (distributed && x.rows > x.cols)
      return err->set(MUON_ERR_SHAPE, who + ": distributed mode shards the long side of a wide matrix; "
                                            "pass a tall matrix transposed (rows <= cols)");
    const int64_t bc = x.cols / k;
    const int64_t lo = distributed ? x.rows : std::min<int64_t>(x.rows, bc);
    const int64_t hi = distributed ? bc : std::max<int64_t>(x.rows, bc);
    if (lo > kMaxMinDim || hi > kMaxMaxDim)
      return err->set(MUON_ERR_SHAPE, who + fmt(": shape %lld x %lld beyond the supported maximum", x.rows, bc));
    if (x.ld > (int64_t(1) << 40) / int64_t(es)) return err->set(MUON_ERR_SHAPE, who + ": ld too large");
    if (reinterpret_cast<uintptr_t>(x.data) % es) return err->set(MUON_ERR_ALIGN, who + ": data not aligned to its element size");
  }
  return true;
}

bool validate_step_triplets(const muon_mat *w, const muon_mat *g, const muon_mat *m, int32_t n, Error *err) {
  for (int32_t i = 0; i < n; ++i) {
    if (g[i].rows != w[i].rows || g[i].cols != w[i].cols || m[i].rows != w[i].rows || m[i].cols != w[i].cols)
      return err->set(MUON_ERR_SHAPE, fmt("matrix %lld: params, grads and moms shapes differ", i));
    if (g[i].dtype != w[i].dtype || m[i].dtype != w[i].dtype)
      return err->set(MUON_ERR_DTYPE, fmt("matrix %lld: params, grads and moms dtypes differ", i));
  }
  return true;
}

bool matrices_overlap(const muon_mat &a, const muon_mat &b) {
  const size_t ea = dtype_size(a.dtype), eb = dtype_size(b.dtype);
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.data), b0 = reinterpret_cast<uintptr_t>(b.data);
  const uintptr_t a1 = a0 + (size_t(a.rows - 1) * a.ld + a.cols) * ea;
  const uintptr_t b1 = b0 + (size_t(b.rows - 1) * b.ld + b.cols) * eb;
  if (a1 <= b0 || b1 <= a0) return false;  // disjoint extents
  // Same pitch and element size: decide exactly on the element grid.
  if (ea != eb || a.ld != b.ld) return true;
  const muon_mat &p = a0 <= b0 ? a : b;  // p starts first
  const muon_mat &q = a0 <= b0 ? b : a;
  const uintptr_t diff = (a0 <= b0 ? b0 - a0 : a0 - b0);
  if (diff % ea) return true;
  const int64_t d = int64_t(diff / ea), ld = p.ld;
  const int64_t qr = d / ld, rc = d % ld;  // q(i, j) sits at p(i + qr, j + rc) while j + rc < ld
  auto rows_meet = [&](int64_t shift) { return shift < p.rows && shift + q.rows > 0; };
  // columns of q that stay on the same p row: j in [0, min(q.cols, ld - rc))
  const int64_t same_hi = std::min<int64_t>(q.cols, ld - rc);
  if (same_hi > 0 && rc < p.cols && rows_meet(qr)) return true;
  // columns of q that wrap onto the next p row: p columns [0, q.cols - (ld - rc))
  const int64_t wrap = q.cols - (ld - rc);
  if (wrap > 0 && rows_meet(qr + 1)) return true;
  return false;
}

bool check_workspace_alias(const muon_mat *const *arrays, const char *const *names, int narrays, int32_t n,
                           const void *ws, size_t ws_bytes, Error *err) {
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(ws), w1 = w0 + ws_bytes;
  for (int a = 0; a < narrays; ++a)
    for (int32_t i = 0; i < n; ++i) {
      const muon_mat &x = arrays[a][i];
      const uintptr_t lo = reinterpret_cast<uintptr_t>(x.data);
      const uintptr_t hi = lo + (size_t(x.rows - 1) * x.ld + x.cols) * dtype_size(x.dtype);
      if (lo < w1 && w0 < hi)
        return err->set(MUON_ERR_ALIAS, std::string(names[a]) + fmt("[%lld] overlaps the workspace", i));
    }
  return true;
}

bool check_alias(const muon_mat *const *arrays, const bool *writable, int narrays, int32_t n, Error *err) {
  struct Item { uintptr_t lo, hi; int arr; int32_t idx; };
  std::vector<Item> items;
  items.reserve(size_t(narrays) * n);
  for (int a = 0; a < narrays; ++a)
    for (int32_t i = 0; i < n; ++i) {
      const muon_mat &x = arrays[a][i];
      const size_t es = dtype_size(x.dtype);
      const uintptr_t lo = reinterpret_cast<uintptr_t>(x.data);
      items.push_back({lo, lo + (size_t(x.rows - 1) * x.ld + x.cols) * es, a, i});
    }
  std::sort(items.begin(), items.end(), [](const Item &x, const Item &y) { return x.lo < y.lo; });
  // Sweep: compare each item with the earlier ones whose extent reaches it.
  std::vector<size_t> active;
  for (size_t k = 0; k < items.size(); ++k) {
    const Item &it = items[k];
    size_t w = 0;
    for (size_t t = 0; t < active.size(); ++t)
      if (items[active[t]].hi > it.lo) active[w++] = active[t];
    active.resize(w);
    for (size_t t : active) {
      const Item &o = items[t];
      if (!writable[it.arr] && !writable[o.arr]) continue;  // read-read sharing is fine
      if (matrices_overlap(arrays[it.arr][it.idx], arrays[o.arr][o.idx]))
        return err->set(MUON_ERR_ALIAS, fmt("buffers overlap (array %lld matrix %lld vs array %lld matrix ",
                                             it.arr, it.idx, o.arr) + std::to_string(o.idx) + ")");
    }
    active.push_back(k);
  }
  return true;
}

bool build_plan(const muon_mat *d, int32_t n, int32_t iters, uint32_t mode, size_t ws_bytes, Plan *plan,
                Error *err) {
  Plan &p = *plan;
  p = Plan{};
  p.iters = iters;
  p.mode = mode;
  p.bf16 = n > 0 ? d[0].dtype == MUON_BF16 : true;
  p.pad = p.bf16 ? kPadBf16 : kPadF32;
  const bool blockwise = mode & MUON_NS_BLOCKWISE;
  p.distributed = mode & MUON_NS_DISTRIBUTED;
  if (p.distributed) {
    // every matrix must have the same shard count: the all-reduce of a
    // launch sums a fixed number of consecutive views
    p.shards = n > 0 ? std::max<int32_t>(d[0].col_blocks, 1) : 1;
    for (int32_t i = 0; i < n; ++i)
      if (std::max<int32_t>(d[i].col_blocks, 1) != p.shards)
        return err->set(MUON_ERR_SHAPE, fmt("distributed mode: matrix %lld has col_blocks %lld, matrix 0 has %lld",
                                            i, int64_t(d[i].col_blocks), int64_t(p.shards)));
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t k = ((blockwise || p.distributed) && d[i].col_blocks > 1) ? d[i].col_blocks : 1;
    const int64_t bc = d[i].cols / k;
    for (int64_t b = 0; b < k; ++b) {
      View v;
      v.mat = i;
      v.block = int32_t(b);
      v.rows = d[i].rows;
      v.cols = bc;
      v.col_off = b * bc;
      // a shard keeps the orientation of its (wide) matrix: X_p is m x n/P
      // even when n/P < m, so that sum_p X_p X_p^T is the Gram of X
      v.tall = p.distributed ? false : v.rows > v.cols;
      v.m = p.distributed ? v.rows : std::min(v.rows, v.cols);
      v.n = p.distributed ? v.cols : std::max(v.rows, v.cols);
      v.mp = round_up(v.m, p.pad);
      v.np = round_up(v.n, p.pad);
      const double m = double(v.m), nn = double(v.n);
      v.cost = double(std::max(iters, 1)) * (4.0 * m * m * nn + 2.0 * m * m * m);
      v.bytes = view_layout(v.mp, v.np, p.bf16, p.distributed).total;
      p.views.push_back(v);
    }
  }
  if (mode & MUON_PACK_COST)
    std::stable_sort(p.views.begin(), p.views.end(), [](const View &a, const View &b) { return a.cost > b.cost; });
  for (const View &v : p.views) {
    p.full_bytes += v.bytes;
    p.min_bytes = std::max(p.min_bytes, v.bytes * size_t(p.shards));  // a matrix's shards go together
  }
  const size_t cap = ws_bytes ? ws_bytes : p.full_bytes;
  if (!p.views.empty() && cap < p.min_bytes)
    return err->set(MUON_ERR_WORKSPACE, fmt("workspace of %lld bytes is smaller than the %lld bytes one matrix needs",
                                            (long long)cap, (long long)p.min_bytes));
  Chunk cur;
  auto flush = [&]() {
    if (cur.count) p.chunks.push_back(cur);
    cur = Chunk{};
  };
  for (int32_t vi = 0; vi < int32_t(p.views.size()); ++vi) {
    const View &v = p.views[vi];
    const bool same_shape = !cur.segs.empty() && cur.segs.back().mp == v.mp && cur.segs.back().np == v.np;
    const bool need_seg = !same_shape;
    // a group starts only at a matrix boundary in distributed mode (the
    // shards of one matrix share their Gram and must be in flight together)
    const bool boundary = !p.distributed || v.block == 0;
    const size_t need = v.bytes * size_t(p.distributed ? p.shards : 1);
    if (boundary && cur.count && (cur.bytes + need > cap || (need_seg && int(cur.segs.size()) == kMaxSegs)))
      flush();
    if (!cur.count) cur.first = vi;
    if (cur.segs.empty() || !(cur.segs.back().mp == v.mp && cur.segs.back().np == v.np)) {
      Segment s;
      s.first = vi;
      s.mp = v.mp;
      s.np = v.np;
      s.base = cur.bytes;
      s.stride = v.bytes;
      const int64_t t = v.mp / kGemmTile;
      if (p.bf16) {
        s.tiles_syrk = t * (t + 1) / 2;
        s.tiles_gemm = t * (v.np / kGemmTile);
      } else {
        const int64_t tf = v.mp / kPadF32;
        s.tiles_syrk = tf * (tf + 1) / 2;
        s.tiles_gemm = tf * (v.np / kPadF32);
      }
      s.tiles_elem = (v.mp / kElemTile) * (v.np / kElemTile);
      cur.segs.push_back(s);
    }
    cur.segs.back().count++;
    cur.count++;
    cur.bytes += v.bytes;
  }
  flush();
  return true;
}

std::string plan_json(const Plan &p) {
  std::ostringstream o;
  o << "{\"bf16\":" << (p.bf16 ? "true" : "false") << ",\"distributed\":" << (p.distributed ? "true" : "false")
    << ",\"shards\":" << p.shards << ",\"pad\":" << p.pad << ",\"iters\":" << p.iters
    << ",\"mode\":" << p.mode << ",\"full_bytes\":" << p.full_bytes << ",\"min_bytes\":" << p.min_bytes
    << ",\"views\":[";
  for (size_t i = 0; i < p.views.size(); ++i) {
    const View &v = p.views[i];
    if (i) o << ",";
    o << "{\"mat\":" << v.mat << ",\"block\":" << v.block << ",\"rows\":" << v.rows << ",\"cols\":" << v.cols
      << ",\"col_off\":" << v.col_off << ",\"tall\":" << (v.tall ? "true" : "false") << ",\"m\":" << v.m
      << ",\"n\":" << v.n << ",\"mp\":" << v.mp << ",\"np\":" << v.np << ",\"cost\":" << v.cost
      << ",\"bytes\":" << v.bytes << "}";
  }
  o << "],\"chunks\":[";
  for (size_t c = 0; c < p.chunks.size(); ++c) {
    const Chunk &ch = p.chunks[c];
    if (c) o << ",";
    int64_t ts = 0, tg = 0, te = 0;
    o << "{\"first\":" << ch.first << ",\"count\":" << ch.count << ",\"bytes\":" << ch.bytes << ",\"segments\":[";
    for (size_t s = 0; s < ch.segs.size(); ++s) {
      const Segment &sg = ch.segs[s];
      if (s) o << ",";
      o << "{\"first\":" << sg.first << ",\"count\":" << sg.count << ",\"mp\":" << sg.mp << ",\"np\":" << sg.np
        << ",\"base\":" << sg.base << ",\"stride\":" << sg.stride << ",\"tiles_syrk\":" << sg.tiles_syrk
        << ",\"tiles_gemm\":" << sg.tiles_gemm;
      const Layout L = view_layout(sg.mp, sg.np, p.bf16, p.distributed);
      o << ",\"layout\":{\"xa\":[" << L.xa[0] << "," << L.xa[1] << "],\"xt\":[" << L.xt[0] << "," << L.xt[1]
        << "],\"ahi\":" << L.ahi << ",\"alo\":" << L.alo << ",\"b\":" << L.b << ",\"bdiag\":" << L.bdiag
        << ",\"partials\":" << L.partials << ",\"tri\":" << L.tri
        << ",\"scale\":" << L.scale << ",\"total\":" << L.total << "}}";
      ts += sg.tiles_syrk * sg.count;
      tg += sg.tiles_gemm * sg.count;
      te += sg.tiles_elem * sg.count;
    }
    o << "],\"launch_tiles\":{\"gram\":" << ts << ",\"aa\":" << ts << ",\"bx\":" << tg << ",\"elem\":" << te
      << "}}";
  }
  o << "]}";
  return o.str();
}

void xcd_ranges(const int64_t *tiles, const int64_t *ksteps, int nseg, int32_t out[9]) {
  double total = 0;
  int64_t count = 0;
  for (int s = 0; s < nseg; ++s) {
    total += double(tiles[s]) * (double(ksteps[s]) + kTileOverheadSteps);
    count += tiles[s];
  }
  out[0] = 0;
  out[8] = int32_t(count);
  for (int x = 1; x < 8; ++x) {
    const double target = total * x / 8;
    double acc = 0;
    int64_t idx = 0;
    for (int s = 0; s < nseg; ++s) {
      const double c = double(ksteps[s]) + kTileOverheadSteps;
      if (acc + double(tiles[s]) * c >= target) {
        idx += std::min<int64_t>(tiles[s], int64_t(std::llround((target - acc) / c)));
        break;
      }
      acc += double(tiles[s]) * c;
      idx += tiles[s];
    }
    out[x] = int32_t(std::min<int64_t>(std::max<int64_t>(idx, out[x - 1]), count));
  }
}

void place(const double *costs, int32_t n, int32_t ranks, uint32_t policy, int32_t *owner,
           double *load) {
  for (int32_t r = 0; r < ranks; ++r) load[r] = 0.0;
  if (policy == MUON_PLACE_RR) {
    for (int32_t i = 0; i < n; ++i) {
      owner[i] = i % ranks;
      load[i % ranks] += costs[i];
    }
    return;
  }
  std::vector<int32_t> order(static_cast<size_t>(n));
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return costs[a] > costs[b]; });
  // min-heap of (load, rank): the least-loaded rank, lower rank on ties
  using Item = std::pair<double, int32_t>;
  std::priority_queue<Item, std::vector<Item>, std::greater<Item>> heap;
  for (int32_t r = 0; r < ranks; ++r) heap.push({0.0, r});
  for (int32_t i : order) {
    Item it = heap.top();
    heap.pop();
    owner[i] = it.second;
    it.first += costs[i];
    load[it.second] = it.first;
    heap.push(it);
  }
}

}  // namespace muon
