// bf16 GEMM instantiation (the fc product: caller's bf16 hidden states times the
// bf16 fc weight, fp32 output), the shared tile / split planner and the launcher.
#include "gemm_dispatch.h"

namespace dfl {

void gemm_dispatch_bf16(EpiKind kind, const GemmPlan& pl, const GemmArgs& g, const void* ep, hipStream_t s) {
  if (kind == EPI_STORE_F32) gemm_cfg<bf16_t, EpiStore<float>>(pl, g, ep, s);
}

GemmPlan plan_gemm(int op, int M, int N, int K, int num_cus, bool wide, bool big_ok) {
  GemmPlan p;
  const bool w16 = op != OP_F32;
  p.bn = 128;
  p.bm = M <= 64 ? 64 : 128;
  // 256 x 256 tiles (one 8-wave work-group per CU) once the grid still holds at
  // least one tile per CU: the injection's fc and K|V products over thousands of
  // rows and the vocabulary product over >= 256 rows (measured: fc 16384 x 4096
  // x 20480 and the 512 x 151936 x 4096 LM head, against 128 x 128 tiles)
  if (w16 && big_ok && M >= 256 && (wide || M >= 2048) &&
      (long)((M + 255) / 256) * ((N + 255) / 256) >= num_cus) {
    p.bm = p.bn = 256;
    return p;
  }
  if (w16 && wide && M <= 64) {
    // the vocabulary product over a few rows (weight streaming): 64 x 128 tiles,
    // 3-deep rings (16 x 151936 x 4096: 231 us, against 240 us for 128 x 128)
    p.bm = 64;
    return p;
  }
  if (w16 && wide) {
    // the vocabulary product: 128 x 128 tiles with a 3-deep weight ring (measured
    // on the 512 x 151936 x 4096 LM head: 743 us, against 1023 us for 128 x 256)
    p.bm = 128;
    p.sb = 3;
    return p;
  }
  if (w16 && K >= 8192 && M > 256 && M <= 768) {
    // long products over a few hundred rows (the MLP down projection): 192 x 128
    // tiles, K split in five (544 x 4096 x 12288 with a plain store: 84 us split
    // in four, against 100 us for 128 x 128 tiles with a 3-deep weight ring); five
    // splits make 480 work-groups for the 512 two-per-CU slots where four left
    // half the CUs with one, and each work-group runs 39 slabs instead of 48;
    // four where five would spill past those slots (the DFlash 2 product's
    // extra correction columns: 540 work-groups)
    p.bm = 192;
    const long t192 = (long)((M + 191) / 192) * ((N + 127) / 128);
    p.splits = t192 * 5 <= 2L * num_cus ? 5 : 4;
    return p;
  }
  if (w16 && K >= 8192 && M > 64 && M <= 1024) {
    // the same products over fewer or more rows: 128 x 128, 3-deep weight ring,
    // K split in four (544 x 4096 x 12288: 101 us, against 120 us for 64 x 128
    // tiles without a split)
    p.sb = 3;
    p.splits = 4;
    return p;
  }
  if (w16 && M > 256 && M <= 768 && N >= 2048 && N <= 4096 && K <= 4096 && N % 64 == 0) {
    // square-ish products over a few hundred rows (the attention output
    // projection): 96 x 64 tiles with 4-deep rings, two or more work-groups
    // per CU (544 x 4096 x 4096 with a plain store: 41.5 us, against 49 us for
    // 64 x 128 tiles)
    p.bm = 96;
    p.bn = 64;
    return p;
  }
  if (w16 && M > 256 && M <= 768 && N <= 1024 && N % 64 == 0) {
    // narrow products over a few hundred rows (the DFlash 2 kernel corrections):
    // 64 x 64 tiles, K split below (544 x 512 x 4096: 17.8 us with a four-way
    // split, against 20.6 us for 64 x 128 tiles)
    p.bm = 64;
    p.bn = 64;
  }
  // 16-bit: 64-row tiles (3 LDS stages, two work-groups per CU) whenever 128-row
  // tiles would leave fewer than two work-groups per CU (measured on the draft's
  // 544-row products: O 66 -> 45 us, down 175 -> 116 us, QKV 69 -> 56 us)
  if (w16 && p.bm == 128 && p.bn == 128 && (long)((M + 127) / 128) * ((N + p.bn - 1) / p.bn) < 2L * num_cus)
    p.bm = 64;
  // up to 64 rows (weight streaming): 64 x 64 tiles with 4-deep rings, K split
  // below (17 rows: QKV 19.4 -> 17.1 us, O 17.2 -> 14.0, gate/up 36.7 -> 33.9,
  // down 26.4 -> 24.5, fc 38.6 -> 33.4 against 64 x 128 tiles; epilogues on whole
  // heads keep 128-wide tiles, see runnable_plan)
  if (w16 && M <= 64 && p.bn == 128 && N % 64 == 0) p.bn = 64;
  const int bk = w16 ? 64 : 32;
  const long tiles = (long)((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
  const int kt = K / bk;
  int sp = 1;
  // Split K for grids far below one work-group per CU (small-M, weight-streaming
  // products), and in two for long products that leave CUs idle; otherwise the
  // partial tiles and their reduction cost more than a partly idle grid (measured).
  if (tiles * 2 < num_cus || (M <= 64 && tiles < 2L * num_cus)) {
    while (tiles * sp * 2 <= 2L * num_cus && kt / (sp * 2) >= 8) sp *= 2;
  } else if (tiles < num_cus && kt >= 192) {
    sp = 2;
  }
  p.splits = sp;
  return p;
}

// The tilings gemm_cfg instantiates for an operand type and epilogue; anything
// else becomes 128 x 128.  The tile counts and split-K partials below are sized
// from the returned plan, so the kernel that runs always matches them.
static GemmPlan runnable_plan(int op, EpiKind kind, GemmPlan p) {
  const bool wide_epi = kind == EPI_QKV || kind == EPI_KVINJECT || kind == EPI_LMHEAD;
  const bool big_epi = kind == EPI_STORE_F32 || kind == EPI_KVINJECT || kind == EPI_LMHEAD;
  if (op == OP_F32) {
    p.bm = p.bm == 64 ? 64 : 128;
    p.bn = 128;
    p.sb = 0;
    return p;
  }
  if (p.bm == 256 && p.bn == 256 && big_epi) {   // the 256 x 256 kernel runs unsplit
    p.splits = 1;
    return p;
  }
  if (p.bn == 128 && (p.bm == 64 || p.bm == 192 || p.bm == 128)) {
    if (p.bm != 128) p.sb = 0;
    return p;
  }
  if (p.bn == 64 && (p.bm == 96 || p.bm == 64)) {
    if (!wide_epi) return p;
    // whole-head / statistics epilogues: the same rows on 128-wide tiles, same K
    // split (17 x 6144 x 4096 with the q/k/v epilogue: split 4 19.4 us, split 8 21.2)
    p.bn = 128;
    if (p.bm == 96) p.bm = 128;
    return p;
  }
  p.bm = p.bn = 128;
  p.sb = 0;
  return p;
}

GemmShape launch_gemm(int op, EpiKind kind, GemmArgs g, const void* epi_params, const GemmPlan& plan_in,
                      float* partials, size_t partials_elems, hipStream_t s) {
  const GemmPlan plan = runnable_plan(op, kind, plan_in);
  const int bk = op != OP_F32 ? 64 : 32;
  g.tiles_m = (g.M + plan.bm - 1) / plan.bm;
  g.tiles_n = (g.N + plan.bn - 1) / plan.bn;
  g.Mpad = g.tiles_m * plan.bm;
  g.Npad = g.tiles_n * plan.bn;
  int splits = plan.splits;
  while (splits > 1 && (size_t)splits * g.Mpad * g.Npad > partials_elems) splits /= 2;
  const int kt = g.K / bk;
  g.splits = splits;
  g.k_per_split = ((kt + splits - 1) / splits) * bk;
  g.partials = partials;
  if (op == OP_F16) gemm_dispatch_f16(kind, plan, g, epi_params, s);
  else if (op == OP_BF16) gemm_dispatch_bf16(kind, plan, g, epi_params, s);
  else gemm_dispatch_f32(kind, plan, g, epi_params, s);
  return GemmShape{g.splits, g.Mpad, g.Npad};
}

}  // namespace dfl
