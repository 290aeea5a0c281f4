// Host driver for the HIP-free validation and planning unit (mla_plan.cpp), built by the CPU test
// suite with a plain host compiler and AddressSanitizer / UndefinedBehaviorSanitizer.
//
//   plan_driver check                      runs the validation cases below, prints one line each
//   plan_driver decode H B max_blocks S    prints the decode plan of a 236B- or Lite-shaped layer
//                                          (H heads) as JSON
//   plan_driver prefill S T max_q max_ctx  prints the prefill plan of the 236B shape (fp8 cache)
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mla.h"
#include "mla_plan.h"

using namespace mla;

namespace {

mla_config base_config(int heads) {
  mla_config c;
  std::memset(&c, 0, sizeof(c));
  c.hidden_size = heads == 16 ? 2048 : 5120;
  c.num_heads = heads;
  c.q_lora_rank = heads == 16 ? 0 : 1536;
  c.kv_lora_rank = 512;
  c.qk_nope_head_dim = 128;
  c.qk_rope_head_dim = 64;
  c.v_head_dim = 128;
  c.page_size = MLA_PAGE_SIZE;
  c.rope_theta = 10000.f;
  c.rms_eps = 1e-6f;
  c.act_dtype = MLA_BF16;
  c.cache_dtype = MLA_BF16;
  c.out_dtype = MLA_F32;
  return c;
}

int failures = 0;
void expect(const char* what, int got, int want) {
  std::printf("%s %s got %d want %d\n", got == want ? "ok" : "FAIL", what, got, want);
  if (got != want) ++failures;
}

// Every region of a plan lies inside [0, bytes) and starts 256-byte aligned; regions are disjoint.
struct Region {
  size_t off, size;
};
void check_regions(const char* what, std::vector<Region> r, size_t bytes) {
  bool good = true;
  for (size_t i = 0; i < r.size(); ++i) {
    if (r[i].off % 256 || r[i].off + r[i].size > bytes) good = false;
    for (size_t j = 0; j < i; ++j)
      if (r[i].size && r[j].size && r[i].off < r[j].off + r[j].size && r[j].off < r[i].off + r[i].size) good = false;
  }
  expect(what, good ? 1 : 0, 1);
}

int run_checks() {
  Dims d;
  Path p;
  mla_config c = base_config(128);
  expect("236B bf16 config", check_config(&c, &d, &p), MLA_OK);
  expect("236B bf16 path", p, PATH_BF16);
  c.cache_dtype = MLA_FP8_E4M3;
  expect("236B fp8 config", check_config(&c, &d, &p), MLA_OK);
  mla_config lite = base_config(16);
  expect("Lite config", check_config(&lite, &d, &p), MLA_OK);
  struct Bad {
    const char* name;
    void (*edit)(mla_config&);
    int status;
  } bad[] = {
      {"null config", nullptr, MLA_ERR_INVALID_ARG},
      {"page size 32", [](mla_config& x) { x.page_size = 32; }, MLA_ERR_INVALID_ARG},
      {"odd rope dim", [](mla_config& x) { x.qk_rope_head_dim = 63; }, MLA_ERR_INVALID_ARG},
      {"zero heads", [](mla_config& x) { x.num_heads = 0; }, MLA_ERR_INVALID_ARG},
      {"act dtype 7", [](mla_config& x) { x.act_dtype = 7; }, MLA_ERR_INVALID_ARG},
      {"cache dtype 9", [](mla_config& x) { x.cache_dtype = 9; }, MLA_ERR_INVALID_ARG},
      {"theta 0", [](mla_config& x) { x.rope_theta = 0.f; }, MLA_ERR_INVALID_ARG},
      {"negative eps", [](mla_config& x) { x.rms_eps = -1.f; }, MLA_ERR_INVALID_ARG},
      {"huge hidden", [](mla_config& x) { x.hidden_size = 1 << 30; }, MLA_ERR_INVALID_ARG},
      {"latent 256", [](mla_config& x) { x.kv_lora_rank = 256; }, MLA_ERR_UNSUPPORTED},
      {"24 heads", [](mla_config& x) { x.num_heads = 24; }, MLA_ERR_UNSUPPORTED},
      {"fp32 act bf16 cache", [](mla_config& x) { x.act_dtype = MLA_F32; }, MLA_ERR_UNSUPPORTED},
      {"yarn without context", [](mla_config& x) { x.rope_factor = 8.f; }, MLA_ERR_INVALID_ARG},
  };
  for (const Bad& b : bad) {
    mla_config x = base_config(128);
    if (b.edit) b.edit(x);
    expect(b.name, check_config(b.edit ? &x : nullptr, nullptr, nullptr), b.status);
  }
  // per-call argument checks: nothing is dereferenced beyond the structs, so dummy addresses do
  c = base_config(128);
  int dummy[4] = {0, 0, 0, 0};
  mla_weights w = {dummy, dummy, dummy, dummy, dummy, dummy};
  mla_cache cache = {dummy, nullptr, 4};
  expect("decode ok", check_decode_args(&c, &w, dummy, dummy, dummy, 4, &cache, 2, 0, dummy), MLA_OK);
  expect("decode null out", check_decode_args(&c, &w, dummy, dummy, dummy, 4, &cache, 2, 0, nullptr),
         MLA_ERR_INVALID_ARG);
  expect("decode 1025 splits", check_decode_args(&c, &w, dummy, dummy, dummy, 4, &cache, 2, 1025, dummy),
         MLA_ERR_INVALID_ARG);
  expect("decode zero batch", check_decode_args(&c, &w, dummy, dummy, dummy, 4, &cache, 0, 0, dummy),
         MLA_ERR_INVALID_ARG);
  mla_weights w_noq = w;
  w_noq.q_a_proj = nullptr;
  expect("decode missing q_a", check_decode_args(&c, &w_noq, dummy, dummy, dummy, 4, &cache, 2, 0, dummy),
         MLA_ERR_INVALID_ARG);
  mla_config f8 = base_config(128);
  f8.cache_dtype = MLA_FP8_E4M3;
  expect("fp8 cache without scales", check_decode_args(&f8, &w, dummy, dummy, dummy, 4, &cache, 2, 0, dummy),
         MLA_ERR_INVALID_ARG);
  expect("prefill ok", check_prefill_args(&c, &w, dummy, dummy, dummy, dummy, 4, &cache, 1, 100, 100, 200, dummy),
         MLA_OK);
  expect("prefill ctx beyond table",
         check_prefill_args(&c, &w, dummy, dummy, dummy, dummy, 4, &cache, 1, 100, 100, 257, dummy), MLA_ERR_INVALID_ARG);
  expect("prefill q longer than tokens",
         check_prefill_args(&c, &w, dummy, dummy, dummy, dummy, 4, &cache, 1, 100, 101, 200, dummy),
         MLA_ERR_INVALID_ARG);
  expect("compress negative count", check_compress_args(&c, &w, dummy, dummy, nullptr, &cache, -1),
         MLA_ERR_INVALID_ARG);
  expect("compress empty", check_compress_args(&c, &w, nullptr, nullptr, nullptr, &cache, 0), MLA_OK);
  // plans: every region aligned, disjoint and inside the workspace
  for (int B : {1, 32, 64, 100, 140}) {
    for (int S : {0, 1, 4, 64}) {
      DecodePlan dp;
      check_config(&c, &d, &p);
      plan_decode(d, p, B, 129, S, &dp);
      const size_t act = 2;
      char what[64];
      std::snprintf(what, sizeof what, "decode regions B=%d S=%d", B, S);
      check_regions(what,
                    {{dp.comp.off_acc, size_t(dp.comp.split.n) * B * d.W() * 4},
                     {dp.q.off_qa_acc, size_t(dp.q.split_a.n) * B * d.dq * 4},
                     {dp.q.off_cq, size_t(B) * d.dq * 4},
                     {dp.q.off_q_acc, size_t(dp.q.split_b.n) * B * d.H * d.dqk() * 4},
                     {dp.off_pos, size_t(B) * 4},
                     {dp.off_slot, size_t(B) * 8},
                     {dp.off_qnope, size_t(B) * d.H * d.dn * act},
                     {dp.off_rope, size_t(B) * d.dr * 4},
                     {dp.off_qhat, size_t(B) * d.H * d.W() * act},
                     {dp.off_part_o, size_t(B) * dp.splits * d.H * d.dc * 2},
                     {dp.off_part_ml, size_t(B) * dp.splits * d.H * 2 * 4},
                     {dp.off_order, size_t(B) * 4},
                     {dp.off_otilde, size_t(B) * d.H * d.dc * 4},
                     {dp.off_ml1, size_t(B) * d.H * 2 * 4}},
                    dp.bytes);
    }
  }
  std::printf("%d failures\n", failures);
  return failures ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc >= 2 && !std::strcmp(argv[1], "check")) return run_checks();
  if (argc == 6 && !std::strcmp(argv[1], "decode")) {
    mla_config c = base_config(std::atoi(argv[2]));
    Dims d;
    Path p;
    if (check_config(&c, &d, &p) != MLA_OK) return 2;
    DecodePlan dp;
    plan_decode(d, p, std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]), &dp);
    std::printf("{\"splits\": %d, \"ordered\": %s, \"cq_pair\": %s, \"hidden_pair\": %s, \"bytes\": %zu}\n",
                dp.splits, dp.ordered ? "true" : "false", dp.cq_pair ? "true" : "false",
                dp.hidden_pair ? "true" : "false", dp.bytes);
    return 0;
  }
  if (argc == 6 && !std::strcmp(argv[1], "prefill")) {
    mla_config c = base_config(128);
    c.cache_dtype = MLA_FP8_E4M3;
    Dims d;
    Path p;
    if (check_config(&c, &d, &p) != MLA_OK) return 2;
    PrefillPlan pp;
    plan_prefill(d, p, std::atoi(argv[2]), std::atoi(argv[3]), std::atoi(argv[4]), std::atoi(argv[5]), 0, &pp);
    std::printf("{\"q16\": %s, \"bytes\": %zu}\n", pp.q16 ? "true" : "false", pp.bytes);
    return 0;
  }
  std::fprintf(stderr, "usage: plan_driver check | decode H B max_blocks splits | prefill S T max_q max_ctx\n");
  return 2;
}
