// Host test of the planner and validation (plan.cpp), built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_plan_host.py.
// plan.cpp has no HIP dependency, so this runs on any machine. A failing
// check prints its expression and line; the program then exits nonzero.
//
// Covered: every validation status of the descriptor checks, the exact
// overlap test and its sweep, the workspace-overlap check, the planner's
// orientation / padding / blockwise and distributed views / cost order /
// grouping under a workspace cap / segment limit / tile counts, the layout
// offsets, the upper-triangle tile enumeration, the RR / LPT placement, and
// the per-XCD tile ranges of persistent launches.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "plan.h"

using namespace muon;

static int g_checks = 0;
#define CHECK(cond)                                                             \
  do {                                                                          \
    ++g_checks;                                                                 \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

static char *fake(uintptr_t k) { return reinterpret_cast<char *>(uintptr_t(1) << 32) + k; }

static muon_mat mat(int64_t r, int64_t c, int32_t dt = MUON_BF16, int64_t ld = 0, char *p = fake(0),
                    int32_t blocks = 1) {
  muon_mat m;
  m.data = p;
  m.rows = r;
  m.cols = c;
  m.ld = ld ? ld : c;
  m.dtype = dt;
  m.col_blocks = blocks;
  return m;
}

static muon_status vd(const std::vector<muon_mat> &d, uint32_t mode = 0) {
  Error e;
  validate_descs(d.data(), int32_t(d.size()), mode, "descs", &e);
  return e.status;
}

static void test_validation() {
  CHECK(vd({}) == MUON_OK);
  {
    Error e;
    CHECK(!validate_descs(nullptr, 1, 0, "d", &e) && e.status == MUON_ERR_INVALID_ARG);
    Error e2;
    CHECK(!validate_descs(nullptr, -1, 0, "d", &e2) && e2.status == MUON_ERR_INVALID_ARG);
  }
  CHECK(vd({mat(4, 8)}) == MUON_OK);
  CHECK(vd({mat(4, 8, 7)}) == MUON_ERR_DTYPE);
  CHECK(vd({mat(4, 8), mat(4, 8, MUON_F32, 0, fake(1 << 20))}) == MUON_ERR_DTYPE);
  CHECK(vd({mat(4, 8, MUON_BF16, 0, nullptr)}) == MUON_ERR_INVALID_ARG);
  CHECK(vd({mat(0, 8)}) == MUON_ERR_SHAPE);
  CHECK(vd({mat(4, -3)}) == MUON_ERR_SHAPE);
  CHECK(vd({mat(4, 8, MUON_BF16, 7)}) == MUON_ERR_SHAPE);
  CHECK(vd({mat(4, 8, MUON_BF16, 0, fake(0), -1)}) == MUON_ERR_SHAPE);
  CHECK(vd({mat(4, 9, MUON_BF16, 0, fake(0), 2)}, MUON_NS_BLOCKWISE) == MUON_ERR_SHAPE);
  CHECK(vd({mat(4, 9, MUON_BF16, 0, fake(0), 2)}) == MUON_OK);  // col_blocks ignored in full mode
  CHECK(vd({mat(40000, 40000)}) == MUON_ERR_SHAPE);
  CHECK(vd({mat(32768, 4194304)}) == MUON_OK);
  CHECK(vd({mat(32769, 4194304)}) == MUON_ERR_SHAPE);
  CHECK(vd({mat(4, 8, MUON_BF16, 0, fake(1))}) == MUON_ERR_ALIGN);
  CHECK(vd({mat(4, 8, MUON_F32, 0, fake(2))}) == MUON_ERR_ALIGN);
  CHECK(vd({mat(9, 8, MUON_BF16, 0, fake(0), 2)}, MUON_NS_DISTRIBUTED) == MUON_ERR_SHAPE);  // tall
  CHECK(vd({mat(4, 8, MUON_BF16, 0, fake(0), 2), mat(4, 8, MUON_BF16, 0, fake(1 << 20), 4)},
           MUON_NS_DISTRIBUTED) == MUON_ERR_SHAPE);
  {
    Error e;
    CHECK(validate_mode(MUON_NS_BLOCKWISE | MUON_PACK_COST | MUON_AA_SPLIT, &e));
    Error e2;
    CHECK(!validate_mode(0x4, &e2) && e2.status == MUON_ERR_INVALID_ARG);
    Error e3;
    CHECK(!validate_mode(MUON_NS_BLOCKWISE | MUON_NS_DISTRIBUTED, &e3) && e3.status == MUON_ERR_INVALID_ARG);
  }
  {
    const muon_mat w[1] = {mat(4, 8)}, g[1] = {mat(4, 8, MUON_BF16, 0, fake(4096))},
                   m[1] = {mat(4, 9, MUON_BF16, 0, fake(8192))};
    Error e;
    CHECK(!validate_step_triplets(w, g, m, 1, &e) && e.status == MUON_ERR_SHAPE);
    const muon_mat m2[1] = {mat(4, 8, MUON_F32, 0, fake(8192))};
    Error e2;
    CHECK(!validate_step_triplets(w, g, m2, 1, &e2) && e2.status == MUON_ERR_DTYPE);
  }
}

static void test_overlap() {
  // two column blocks of one 8 x 64 bf16 buffer interleave without sharing
  // an element; a shift by one element makes them meet
  const muon_mat left = mat(8, 32, MUON_BF16, 64, fake(0));
  const muon_mat right = mat(8, 32, MUON_BF16, 64, fake(64));
  const muon_mat shifted = mat(8, 32, MUON_BF16, 64, fake(62));
  CHECK(!matrices_overlap(left, right));
  CHECK(matrices_overlap(left, shifted));
  CHECK(!matrices_overlap(left, mat(8, 32, MUON_BF16, 64, fake(16 * 64 * 2))));  // after the last row
  CHECK(matrices_overlap(left, mat(1, 1, MUON_BF16, 1, fake(7 * 128 + 62))));    // last element
  CHECK(!matrices_overlap(left, mat(1, 1, MUON_BF16, 1, fake(7 * 128 + 64))));   // just past it, in the gap
  // brute force on a small grid of placements and pitches
  for (int ld = 3; ld <= 6; ++ld)
    for (int off = 0; off < 40; ++off)
      for (int rows = 1; rows <= 3; ++rows)
        for (int cols = 1; cols <= ld; ++cols) {
          const muon_mat a = mat(3, 2, MUON_F32, ld, fake(0));
          const muon_mat b = mat(rows, cols, MUON_F32, ld, fake(size_t(off) * 4));
          bool hit = false;
          for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 2; ++j)
              for (int p = 0; p < rows; ++p)
                for (int q = 0; q < cols; ++q) hit |= (i * ld + j) == (off + p * ld + q);
          CHECK(matrices_overlap(a, b) == hit);
          CHECK(matrices_overlap(b, a) == hit);
        }
  // the sweep: read-read sharing passes, a written overlap does not
  const muon_mat g[2] = {mat(4, 8, MUON_BF16, 0, fake(0)), mat(4, 8, MUON_BF16, 0, fake(0))};
  const muon_mat w[2] = {mat(4, 8, MUON_BF16, 0, fake(4096)), mat(4, 8, MUON_BF16, 0, fake(8192))};
  const muon_mat *arrays[2] = {w, g};
  const bool wr[2] = {true, false};
  Error e;
  CHECK(check_alias(arrays, wr, 2, 2, &e));
  const muon_mat w2[2] = {mat(4, 8, MUON_BF16, 0, fake(4096)), mat(4, 8, MUON_BF16, 0, fake(4096 + 60))};
  const muon_mat *arrays2[2] = {w2, g};
  Error e2;
  CHECK(!check_alias(arrays2, wr, 2, 2, &e2) && e2.status == MUON_ERR_ALIAS);
  // the workspace
  const char *names[2] = {"params", "grads"};
  Error e3;
  CHECK(check_workspace_alias(arrays, names, 2, 2, fake(1 << 20), 4096, &e3));
  Error e4;
  CHECK(!check_workspace_alias(arrays, names, 2, 2, fake(8192 + 63), 16, &e4) && e4.status == MUON_ERR_ALIAS);
  CHECK(e4.msg.find("params[1]") != std::string::npos);
  Error e5;
  CHECK(check_workspace_alias(arrays, names, 2, 2, fake(8192 + 64), 16, &e5));  // ends where it starts
}

static void test_plan() {
  // orientation, padding, cost and order
  std::vector<muon_mat> d = {mat(300, 520, MUON_BF16, 0, fake(0)), mat(520, 300, MUON_BF16, 0, fake(1 << 20)),
                             mat(256, 256, MUON_BF16, 0, fake(2 << 20)), mat(1, 7, MUON_BF16, 0, fake(3 << 20))};
  Plan p;
  Error e;
  CHECK(build_plan(d.data(), 4, 5, MUON_PACK_RR, 0, &p, &e));
  CHECK(p.views.size() == 4 && p.chunks.size() == 1);
  CHECK(!p.views[0].tall && p.views[1].tall && !p.views[2].tall);
  CHECK(p.views[0].m == 300 && p.views[0].n == 520 && p.views[0].mp == 512 && p.views[0].np == 768);
  CHECK(p.views[1].m == 300 && p.views[1].n == 520);
  CHECK(p.views[3].mp == 256 && p.views[3].np == 256);
  CHECK(p.views[0].cost == 5.0 * (4.0 * 300 * 300 * 520 + 2.0 * 300 * 300 * 300));
  Plan pc;
  CHECK(build_plan(d.data(), 4, 5, MUON_PACK_COST, 0, &pc, &e));
  for (size_t i = 1; i < pc.views.size(); ++i) CHECK(pc.views[i - 1].cost >= pc.views[i].cost);
  CHECK(pc.views[0].mat == 0 && pc.views[1].mat == 1);  // equal costs keep the given order
  // segments: consecutive views of one padded shape share a segment
  CHECK(pc.chunks[0].segs.size() == 2);  // 512 x 768 twice, then 256 x 256 twice
  CHECK(pc.chunks[0].segs[1].count == 2 && pc.chunks[0].segs[1].tiles_syrk == 1);
  CHECK(pc.chunks[0].segs[0].count == 2 && pc.chunks[0].segs[0].tiles_syrk == 3 &&
        pc.chunks[0].segs[0].tiles_gemm == 2 * 3);
  // workspace cap: views are grouped into chunks that fit it
  const size_t one = pc.views[0].bytes;
  Plan pg;
  CHECK(build_plan(d.data(), 4, 5, MUON_PACK_COST, one, &pg, &e));
  CHECK(pg.chunks.size() >= 2);
  for (const Chunk &c : pg.chunks) CHECK(c.bytes <= one || c.count == 1);
  Error ew;
  Plan ps;
  CHECK(!build_plan(d.data(), 4, 5, MUON_PACK_COST, one - 256, &ps, &ew) && ew.status == MUON_ERR_WORKSPACE);
  // layout: every buffer of a view inside its block, 256-byte aligned
  const Layout L = view_layout(512, 768, true, true);
  const size_t offs[] = {L.xa[0], L.xa[1], L.xt[0], L.xt[1], L.ahi, L.alo, L.b, L.bdiag, L.partials, L.scale, L.tri};
  for (size_t o : offs) CHECK(o % 256 == 0 && o < L.total);
  CHECK(L.xa[1] - L.xa[0] == size_t(512) * 768 * 2 && L.nparts == (512 / 64) * (768 / 64));
  CHECK(L.total - L.tri >= size_t(512) * 513 / 2 * 4);
  // blockwise: each block is its own view, oriented on its own
  std::vector<muon_mat> b = {mat(7168, 18432, MUON_BF16, 0, fake(0), 8)};
  Plan pb;
  CHECK(build_plan(b.data(), 1, 5, MUON_NS_BLOCKWISE, 0, &pb, &e));
  CHECK(pb.views.size() == 8);
  for (int k = 0; k < 8; ++k) {
    CHECK(pb.views[k].col_off == 2304 * k && pb.views[k].tall);
    CHECK(pb.views[k].m == 2304 && pb.views[k].n == 7168 && pb.views[k].mp == 2304 && pb.views[k].np == 7168);
  }
  // distributed: shards keep the matrix's orientation; a chunk holds whole matrices
  std::vector<muon_mat> s = {mat(512, 2048, MUON_BF16, 0, fake(0), 4), mat(512, 2048, MUON_BF16, 0, fake(4 << 20), 4)};
  Plan pd;
  CHECK(build_plan(s.data(), 2, 5, MUON_NS_DISTRIBUTED, 0, &pd, &e));
  CHECK(pd.distributed && pd.shards == 4 && pd.views.size() == 8);
  CHECK(pd.views[0].m == 512 && pd.views[0].n == 512 && !pd.views[0].tall);
  Plan pd2;
  CHECK(build_plan(s.data(), 2, 5, MUON_NS_DISTRIBUTED, pd.views[0].bytes * 4, &pd2, &e));
  CHECK(pd2.chunks.size() == 2 && pd2.chunks[0].count == 4 && pd2.chunks[1].count == 4);
  // more than kMaxSegs distinct shapes: a new chunk starts
  std::vector<muon_mat> many;
  for (int k = 0; k < 10; ++k) many.push_back(mat(256 * (k + 1), 2560, MUON_BF16, 0, fake(size_t(k) << 24)));
  Plan pm;
  CHECK(build_plan(many.data(), 10, 5, MUON_PACK_RR, 0, &pm, &e));
  CHECK(pm.chunks.size() == 2 && pm.chunks[0].segs.size() == size_t(kMaxSegs));
  // float32 path pads to 64
  std::vector<muon_mat> f = {mat(64, 128, MUON_F32)};
  Plan pf;
  CHECK(build_plan(f.data(), 1, 5, 0, 0, &pf, &e));
  CHECK(!pf.bf16 && pf.views[0].mp == 64 && pf.views[0].np == 128);
  const std::string js = plan_json(pc);
  CHECK(js.find("\"views\":[") != std::string::npos && js.find("\"launch_tiles\"") != std::string::npos);
}

static void test_tiles_and_place() {
  int64_t u = 0;
  for (int64_t J = 0; J < 40; ++J)
    for (int64_t I = 0; I <= J; ++I, ++u) {
      int64_t a, b;
      syrk_tile(u, &a, &b);
      CHECK(a == I && b == J);
    }
  const double costs[7] = {5, 5, 4, 4, 3, 3, 3};
  int32_t owner[7];
  double load[3];
  place(costs, 7, 3, MUON_PLACE_RR, owner, load);
  for (int i = 0; i < 7; ++i) CHECK(owner[i] == i % 3);
  CHECK(load[0] == 5 + 4 + 3 && load[1] == 5 + 3 && load[2] == 4 + 3);
  place(costs, 7, 3, MUON_PLACE_LPT, owner, load);
  // Graham's tight example: LPT gives 11 where 9 is optimal
  double mx = 0;
  for (int r = 0; r < 3; ++r) mx = load[r] > mx ? load[r] : mx;
  CHECK(mx == 11);
  CHECK(owner[0] == 0 && owner[1] == 1 && owner[2] == 2);
}

// Per-XCD tile ranges of a persistent launch: contiguous, monotone, covering
// every tile; equal tile costs give the count split (to within one tile);
// mixed K gives each XCD about an eighth of the estimated time.
static std::vector<int32_t> check_ranges(const std::vector<int64_t> &tiles, const std::vector<int64_t> &ksteps) {
  int32_t r[9];
  xcd_ranges(tiles.data(), ksteps.data(), int(tiles.size()), r);
  int64_t n = 0;
  double total = 0, biggest = 0;
  std::vector<double> cost;
  for (size_t s = 0; s < tiles.size(); ++s) {
    const double c = double(ksteps[s]) + kTileOverheadSteps;
    n += tiles[s];
    for (int64_t t = 0; t < tiles[s]; ++t) cost.push_back(c);
    total += double(tiles[s]) * c;
    if (tiles[s] && c > biggest) biggest = c;
  }
  CHECK(r[0] == 0 && r[8] == n);
  double worst = 0;
  for (int x = 0; x < 8; ++x) {
    CHECK(r[x] <= r[x + 1]);
    double c = 0;
    for (int32_t t = r[x]; t < r[x + 1]; ++t) c += cost[size_t(t)];
    worst = c > worst ? c : worst;
  }
  CHECK(worst <= total / 8 + biggest + 1e-9);  // at most one tile above an even split
  return std::vector<int32_t>(r, r + 9);
}

static void test_xcd_ranges() {
  // uniform: the count split
  const auto u = check_ranges({1152 * 224}, {64});
  for (int x = 0; x <= 8; ++x) CHECK(std::llabs(int64_t(u[size_t(x)]) - int64_t(1152) * 224 * x / 8) <= 1);
  // a Qwen3-block-like B X launch: 256 tiles of 64 K steps first, then 32
  // of 16 and 9216 of 24; split by count, the first XCD would get all the
  // long tiles and 17% more than an eighth of the time
  const auto m = check_ranges({256, 32, 9216}, {64, 16, 24});
  CHECK(m[1] < 9504 / 8);
  check_ranges({3, 1, 5}, {128, 8, 24});  // fewer tiles than XCDs
  check_ranges({0, 40}, {64, 24});        // an empty segment
}

int main() {
  test_validation();
  test_overlap();
  test_plan();
  test_tiles_and_place();
  test_xcd_ranges();
  std::printf("plan host test: %d checks passed\n", g_checks);
  return 0;
}
