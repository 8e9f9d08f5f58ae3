// Host-side exercise of libzo's runtime (zo_api.cpp) for the AddressSanitizer and
// UndefinedBehaviorSanitizer build: plan validation, packing, workspace carving, bank
// geometry and keys, the estimate and the error paths of every call, on many seeded
// random batches and plans.  Nothing here launches a kernel (no GPU is needed): the
// calls either stay on the host or return an error before any launch.  Exit status 0
// and no sanitizer report means the host arithmetic stayed in bounds and defined.
#include "../../include/zo.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

namespace {

int g_fail = 0;
#define EXPECT(cond)                                                             \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (%s)\n", __FILE__,      \
                   __LINE__, #cond, zo_last_error());                            \
      ++g_fail;                                                                  \
    }                                                                            \
  } while (0)

zo_model_desc opt_desc(int layers, int d, int heads, int ffn, int vocab, int dtype) {
  zo_model_desc m;
  std::memset(&m, 0, sizeof m);
  m.abi_version = ZO_ABI_VERSION;
  m.arch = ZO_ARCH_OPT;
  m.dtype = dtype;
  m.n_layers = layers; m.d_model = d; m.n_heads = heads; m.n_kv_heads = heads; m.head_dim = d / heads;
  m.d_ffn = ffn; m.vocab = vocab; m.max_pos = 2048; m.norm_eps = 1e-5; m.rope_theta = 0;
  return m;
}

struct Batch {
  std::vector<int32_t> cu, role, mode;
  zo_batch b;
};

Batch random_batch(std::mt19937& rs, int max_seq, int max_len) {
  Batch B;
  const int n = std::uniform_int_distribution<int>(0, max_seq)(rs);
  B.cu.assign(1, 0);
  for (int i = 0; i < n; ++i) {
    const int len = std::uniform_int_distribution<int>(2, max_len)(rs);
    B.cu.push_back(B.cu.back() + len);
    B.role.push_back(std::uniform_int_distribution<int>(0, 1)(rs));
    B.mode.push_back(std::uniform_int_distribution<int>(0, 1)(rs));
  }
  B.b.n_seq = n;
  B.b.cu_seqlens = B.cu.data();
  B.b.tokens_dev = (const int32_t*)(uintptr_t)0x1000;   // never dereferenced on these paths
  B.b.role = B.role.empty() ? nullptr : B.role.data();
  B.b.score_mode = B.mode.empty() ? nullptr : B.mode.data();
  if (n == 0) { static int32_t dummy = 0; B.b.role = &dummy; B.b.score_mode = &dummy; }
  return B;
}

}  // namespace

int main() {
  std::mt19937 rs(20261203u);
  const zo_model_desc descs[] = {opt_desc(2, 128, 4, 512, 512, ZO_DTYPE_F32),
                                 opt_desc(3, 256, 4, 512, 1000, ZO_DTYPE_BF16),
                                 opt_desc(2, 256, 4, 512, 1000, ZO_DTYPE_FP8)};
  for (const zo_model_desc& md : descs) {
    size_t wbytes = 0;
    EXPECT(zo_weights_size(&md, &wbytes) == ZO_OK && wbytes > 0);
    for (int slot = 0; slot <= md.n_layers; ++slot)
      for (int param = -1; param < 20; ++param) {
        size_t off; int64_t rows, cols; int32_t dt, lay;
        const int rc = zo_weight_locate(&md, slot, param, &off, &rows, &cols, &dt, &lay);
        EXPECT(rc == ZO_OK || rc == ZO_E_INVAL);
        if (rc == ZO_OK) EXPECT(off < wbytes && rows > 0 && cols > 0);
      }
    zo_model* m = nullptr;
    EXPECT(zo_model_create(&md, (void*)(uintptr_t)0x10000, wbytes, &m) == ZO_OK);
    if (!m) return 1;
    for (int trial = 0; trial < 300; ++trial) {
      const int rank = std::uniform_int_distribution<int>(1, 8)(rs);
      const int q = std::uniform_int_distribution<int>(1, 4)(rs);
      std::vector<uint64_t> seeds;
      for (int i = 0; i < q; ++i) seeds.push_back(1000u * trial + 7u * i + 1u);
      std::vector<int32_t> cdir, csign;
      for (int i = 0; i < q; ++i) { cdir.push_back(i); csign.push_back(1); cdir.push_back(i); csign.push_back(-1); }
      zo_plan_desc pd;
      std::memset(&pd, 0, sizeof pd);
      pd.step = (uint64_t)std::uniform_int_distribution<int>(0, 50)(rs);
      pd.nu = (uint32_t)std::uniform_int_distribution<int>(1, 6)(rs);
      pd.rank = rank; pd.eps = 1e-3; pd.n_dirs = q; pd.dir_seeds = seeds.data();
      pd.n_cand = (int32_t)cdir.size(); pd.cand_dir = cdir.data(); pd.cand_sign = csign.data();
      pd.target_mask = (uint32_t)std::uniform_int_distribution<int>(0, 63)(rs);
      pd.flags = (trial % 5 == 0 && md.dtype == ZO_DTYPE_BF16) ? ZO_PLAN_ACT_SPLIT : 0u;
      zo_plan_t* p = nullptr;
      EXPECT(zo_plan(m, &pd, &p) == ZO_OK);
      if (!p) continue;
      // bank with random keys: some slots empty, some frozen, some of the plan's window
      const int n_slots = std::uniform_int_distribution<int>(1, 6)(rs);
      size_t bbytes = 0;
      EXPECT(zo_bank_size(m, n_slots, rank, pd.target_mask, &bbytes) == ZO_OK);
      zo_bank* bank = nullptr;
      EXPECT(zo_bank_create(m, n_slots, rank, pd.target_mask, (void*)(uintptr_t)0x20000, bbytes, &bank) == ZO_OK);
      std::vector<uint64_t> ks(n_slots);
      std::vector<int64_t> kw(n_slots);
      for (int s = 0; s < n_slots; ++s) {
        ks[s] = seeds[std::uniform_int_distribution<int>(0, q - 1)(rs)];
        kw[s] = std::uniform_int_distribution<int>(-1, 8)(rs);
      }
      EXPECT(zo_bank_set_keys(bank, ks.data(), kw.data()) == ZO_OK);
      for (int s = 0; s < n_slots; ++s)
        for (int l = 0; l < md.n_layers; ++l)
          for (int k = 0; k < 7; ++k) {
            size_t off;
            const int rc = zo_bank_entry_offset(bank, s, l, k, &off);
            if (rc == ZO_OK) EXPECT(off + sizeof(float) <= bbytes);
          }
      Batch B = random_batch(rs, 12, 150);
      int32_t n_phys = 0;
      int64_t n_rows = 0, n_sc = 0;
      size_t ws = 0;
      const int rc = zo_batch_layout(m, p, bank, &B.b, &n_phys, &n_rows, &n_sc, &ws);
      EXPECT(rc == ZO_OK || rc == ZO_E_SHAPE);
      if (rc == ZO_OK) {
        std::vector<int32_t> ps(n_phys + 1), pc(n_phys + 1), pf(n_phys + 1);
        EXPECT(zo_pack(p, &B.b, ps.data(), pc.data(), pf.data()) == ZO_OK);
        EXPECT(pf[n_phys] == n_sc);
        // a workspace one byte short is refused before any launch
        std::vector<double> S(pd.n_cand);
        if (ws > 0)
          EXPECT(zo_score(m, p, bank, &B.b, (void*)(uintptr_t)0x30000, ws - 1, nullptr, nullptr, S.data(), nullptr) ==
                 ZO_E_SHAPE);
        int32_t gp = 0;
        size_t gws = 0;
        const int grc = zo_generate_layout(m, p, bank, &B.b, 3, &gp, &gws);
        EXPECT(grc == ZO_OK || grc == ZO_E_INVAL || grc == ZO_E_SHAPE);
      }
      // estimate on random scores, with and without the flags
      std::vector<double> S(pd.n_cand), c(q);
      std::vector<int64_t> nsc(pd.n_cand, 7);
      for (double& v : S) v = -std::uniform_real_distribution<double>(0, 50)(rs);
      for (uint32_t f = 0; f < 4; ++f) EXPECT(zo_estimate(p, S.data(), nsc.data(), f, c.data()) == ZO_OK);
      S[0] = 0.0 / 0.0;
      EXPECT(zo_estimate(p, S.data(), nullptr, 0, c.data()) == ZO_E_NONFINITE);
      // a cap with nothing to fold touches no device memory
      int32_t nf = -1;
      int cap_rc = zo_bank_cap(m, bank, p, n_slots, nullptr, 0, nullptr, &nf);
      EXPECT(cap_rc == ZO_OK && nf == 0);
      zo_bank_destroy(bank);
      zo_plan_destroy(p);
    }
    // invalid descriptors and arguments
    zo_plan_desc bad;
    std::memset(&bad, 0, sizeof bad);
    zo_plan_t* p = nullptr;
    EXPECT(zo_plan(m, &bad, &p) == ZO_E_INVAL);
    EXPECT(zo_score_noalloc(m, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == ZO_E_INVAL);
    zo_model_destroy(m);
  }
  zo_model_desc broken = opt_desc(2, 130, 4, 512, 512, ZO_DTYPE_BF16);   // head_dim 32.5
  size_t n = 0;
  EXPECT(zo_weights_size(&broken, &n) != ZO_OK);
  std::printf("host driver: %d failed expectations\n", g_fail);
  return g_fail ? 1 : 0;
}
