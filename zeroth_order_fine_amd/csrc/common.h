// Internal declarations shared by the HIP translation units of libzo.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef uint16_t bf16_t;   // storage type: raw bf16 bits

// ---- bf16 helpers (round to nearest even; inputs are finite) ---------------
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  uint32_t lsb = (u >> 16) & 1u;
  return (bf16_t)((u + 0x7FFFu + lsb) >> 16);
}
__host__ __device__ inline float bf16_to_f32(bf16_t b) {
  return __builtin_bit_cast(float, ((uint32_t)b) << 16);
}
// two fp32 values rounded to bf16 (nearest even, as f32_to_bf16) by the packed hardware
// conversion, packed little-endian; and back
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2v_t{(__bf16)a, (__bf16)b});
}
__device__ inline float bf16x2_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16x2_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
// Two-term bf16 expansion of an fp32 value: hi = bf16(v), lo = bf16(v - hi).
// v - hi is exact in fp32, so hi + lo carries 16 significant bits (relative
// error <= 2^-17); a product with an exact bf16 weight then needs two MFMAs.
__host__ __device__ inline void split_bf16(float v, bf16_t& hi, bf16_t& lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - bf16_to_f32(hi));
}

// activation element type helpers: float (fp32 mode) or bf16_t (bf16 mode)
template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// ---- OCP e4m3 (fp8 models) ----------------------------------------------------
// e4m3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities, largest
// finite magnitude 448.  fp8 models store their layer linears as e4m3 codes of w * 2^11
// and feed those linears e4m3 activations.
typedef uint8_t e4m3_t;
constexpr int ZO_FP8_WEIGHT_EXP = 11;
// four fp32 values -> four e4m3 codes, packed little-endian (value 0 in the low byte):
// round to nearest even (the hardware conversion), magnitudes clamped to 448 first,
// so an overflow saturates instead of producing NaN
__device__ inline uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  auto cl = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
  return (uint32_t)w;
}
// eight e4m3 codes (little-endian in two words) -> eight bf16 (exact: every e4m3 value
// is a bf16 value)
__device__ inline u32x4_t e4m3x8_to_bf16(uint2 v) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_v;
  const bf16x2_v p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, false);
  const bf16x2_v p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, true);
  const bf16x2_v p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, false);
  const bf16x2_v p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, true);
  return u32x4_t{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
}

// ---- GEMM -------------------------------------------------------------------
// C[M x N] = A[M x K] . B[N x K]^T  (+ side: As[M x Ks] . Bs[N x Ks]^T), fused epilogue.
enum GemmEpi {
  EPI_STORE = 0,    // C = act(acc + bias), activation-typed output
  EPI_GELU = 1,     // C = gelu_erf(acc + bias)
  EPI_SWIGLU = 2,   // packed gate/up (16-column interleave): C[:, j] = silu(gate_j) * up_j
  EPI_RESID = 3,    // H (fp32) += acc + bias
  EPI_TPROJ = 4,    // side-input builder: columns of x.[V...] scattered by candidate
  EPI_LMHEAD = 5,   // per row and column tile: (max, sum exp) and the label logit
  EPI_PARTIAL = 6,  // split-K: fp32 partial sums of one K-slice (blockIdx.z) to `partial`
};

struct GemmParams {
  const void* A; int64_t lda;
  const void* B; int64_t ldb;
  int M, N, K;
  // Column wraps of the main segment (0: none): K-step k reads A column k mod kwa
  // and B column k mod kwb (k < 2 * wrap).  With two-term bf16 activations
  // A = [hi | lo], K = 2 kwb: hi.W^T + lo.W^T in one pass over the exact bf16 W;
  // with B = [V_hi | V_hi | V_lo], K = 3 kwa: hi.V_hi + lo.V_hi + hi.V_lo.
  int kwa, kwb;
  // extended-K side path (0 = none). Column tile starting at n0 uses the
  // As columns [g*ks_tile, (g+1)*ks_tile) where g = number of bounds <= n0.
  const void* As; int64_t ldas;
  const void* Bs; int64_t ldbs;
  int ks_tile;
  int n_bounds; int bounds[3];
  int as_stride;              // As columns per group (0: ks_tile)
  int kwas;                   // side-segment As column wrap (0: none), as kwa

  // epilogue
  int epi;
  const float* bias;          // [N] or null
  void* C; int64_t ldc;       // STORE/GELU/SWIGLU/TPROJ output
  int c_lo;                   // bf16 outputs: 0, or write the two-term expansion with lo at column + c_lo
  int c_f32;                  // STORE of the bf16 kernels: write fp32 instead of bf16
  float* H; int64_t ldh;      // RESID target
  // TPROJ
  const int32_t* row_cand;    // [M] candidate or -1
  const int32_t* cand_dir;    // [n_cand]
  const int32_t* cand_slot;   // [n_cand] computed t slot of the candidate's direction
  const float* cand_scale;    // [n_cand] sign * eps_tilde
  int tp_ks;                  // computed columns per kind block (nc * r, padded)
  int tp_rank;                // r
  int tp_entries;             // E active bank entries (computed slots and As blocks before the directions)
  int tp_used;                // nc * r computed columns per kind block
  int tp_as_ks;               // As columns per kind block ((E + q) * r, padded)
  int tp_unit;                // 0, or write t as two-term bf16: column c of unit u = c / tp_unit goes to
                              // u * 2 tp_unit + c % tp_unit (hi) and + tp_unit more (lo)
  // LMHEAD
  const int32_t* labels;      // [M]
  float2* part;               // [M x n_ntiles]
  float* lab_logit;           // [M]
  int n_ntiles;
  int32_t* part_idx;          // null, or [M x n_ntiles]: first column holding the tile's row maximum (greedy decoding)
  // split-K (EPI_PARTIAL): K-slice z covers base K-steps [z*ksteps_per_split, ...)
  int ksplit;
  float* partial;             // [ksplit x M x N]
  // fp8 models: a_e4m3 = A holds e4m3 codes; b_e4m3 = B holds e4m3 codes of w * 2^11
  // (the projection kernel then runs the main segment as e4m3 x e4m3 MFMAs, takes the
  // side segment's Bs pre-scaled by 2^11, multiplies the sums by 2^-11 before the
  // epilogue, and writes GELU outputs as e4m3)
  int a_e4m3, b_e4m3;
  // GELU / SwiGLU epilogues (bf16 kernels): the side input of the projection that reads this
  // output, formed here (sf_n used factor columns, 0 = none).  Per row and group of the
  // output columns two adjacent wave tiles hold (128 for GELU, 64 for SwiGLU), the partial
  // sums of the stored (rounded) outputs times the used V^T rows: column j of sf_n is row
  // (j / sf_used) * sf_ks + j % sf_used of sf_vt (row pitch sf_ldv), written to
  // sf_part [M x sf_groups x sf_n] fp32; side_part_reduce sums each row's groups.
  int sf_n, sf_used, sf_ks, sf_groups;
  const void* sf_vt; int64_t sf_ldv;
  float* sf_part;
  // Split tail of the 256x256 projection kernel (null: off).  A launch of sk_ncu persistent
  // workgroups (one per CU) runs the last one to two rounds of tiles in K-slices dealt out
  // evenly; slice j of a tile leaves its fp32 accumulators in the tile's sk_part buffer
  // (256 x 256 floats; two buffers per workgroup) and sets the tile's sk_flag word to
  // j + 1; slice j + 1 waits for it, continues the same K sequence from those accumulators
  // and the last slice clears the word (the words are zero between launches).  sk_flag
  // holds 2 ZO_SK_MAX_WG flag words, then ZO_SK_MAX_WG words for the XCD each workgroup
  // ran on.  sk_err is set to 1 if a wait ever gives up, to 2 if a handover crossed XCDs.
  float* sk_part;
  int32_t* sk_flag;
  int32_t* sk_err;
  int sk_ncu;
};
// split-tail workgroups a workspace provides for (one per CU, at most; two buffers each)
constexpr int ZO_SK_MAX_WG = 256;

// Launch on `stream`; returns hipSuccess or the launch error.
hipError_t gemm_launch_bf16(const GemmParams& p, int cfg, hipStream_t stream);
hipError_t gemm_launch_f32(const GemmParams& p, int cfg, hipStream_t stream);
enum GemmCfg { GEMM_CFG_BIG = 0, GEMM_CFG_NARROW = 1, GEMM_CFG_HEAD = 2 };
int gemm_cfg_bn(int cfg, bool bf16);
int gemm_cfg_bm(int cfg, bool bf16);
int gemm_bk(bool bf16);
int gemm_cfg_bk(int cfg, bool bf16);

// ---- side input t: the As columns a row's candidate state needs -----------------
// Shared by the side-input projections (gemm.hip) and the norm kernel that forms t for the
// projections reading its output (layers.hip).
template <typename TAct>
__device__ __forceinline__ void store_tproj(const GemmParams& p, int r, int c, float v);

// Side input of row r from computed column c = x.V (kind block c / tp_ks, computed
// slot (c % tp_ks) / r): a bank entry's slot goes to the entry's As block; the slot
// of the row's own direction also goes, times s * eps~, to that direction's As
// block.  Nothing else is written (As is zero-filled once per call; foreground rows
// and other directions keep zeros).
template <typename TAct>
__device__ __forceinline__ void tproj_out(const GemmParams& p, int r, int c, float v, int cand) {
  if (cand < 0) return;
  const int kb = c / p.tp_ks, w = c - kb * p.tp_ks;
  if (w >= p.tp_used) return;
  const int slot = w / p.tp_rank, k = w - slot * p.tp_rank;
  const int base = kb * p.tp_as_ks + k;
  if (slot < p.tp_entries) store_tproj<TAct>(p, r, base + slot * p.tp_rank, v);
  if (slot == p.cand_slot[cand])
    store_tproj<TAct>(p, r, base + (p.tp_entries + p.cand_dir[cand]) * p.tp_rank, p.cand_scale[cand] * v);
}

// side input t of row r, As column c (see tp_unit)
template <typename TAct>
__device__ __forceinline__ void store_tproj(const GemmParams& p, int r, int c, float v) {
  if constexpr (std::is_same<TAct, float>::value) {
    ((float*)p.C)[(int64_t)r * p.ldc + c] = v;
  } else {
    if (p.tp_unit == 0) {
      ((bf16_t*)p.C)[(int64_t)r * p.ldc + c] = f32_to_bf16(v);
      return;
    }
    const int u = c / p.tp_unit;
    const int64_t o = (int64_t)r * p.ldc + c + u * p.tp_unit;   // u * 2 tp_unit + c % tp_unit
    bf16_t hi, lo;
    split_bf16(v, hi, lo);
    ((bf16_t*)p.C)[o] = hi;
    ((bf16_t*)p.C)[o + p.tp_unit] = lo;
  }
}


// ---- random streams ---------------------------------------------------------
struct NormalJob {     // one generated tensor (or factor) written in a given layout
  void* dst;           // output base
  int64_t rows, cols;  // logical shape; element e = row*cols + col of the stream
  int64_t ld;          // physical row pitch (elements)
  uint64_t seed; uint64_t tau; uint32_t tag;
  int32_t mode;        // see rng.hip
  int32_t dtype;       // 0 f32, 1 bf16, 2 e4m3 code of v * 2^11
  int32_t pad_;
  int64_t aux;         // mode specific
};
hipError_t launch_normal_jobs(const NormalJob* jobs_dev, int n_jobs, int64_t max_blocks, hipStream_t s);
hipError_t launch_normal_fill_f64(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first, int64_t n,
                                  double* out, hipStream_t s);
hipError_t launch_words_fill(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first_block, int64_t n_blocks,
                             uint32_t* out, hipStream_t s);

struct SideJob {       // one side-path factor block of one target linear
  void* dst; int64_t ld;          // destination (Vt rows or Bs rows)
  const float* u_src;             // bank U [n_out x r] (SRC_BANK) or null
  uint64_t seed; uint64_t tau; uint32_t tag;
  int32_t src;                    // 0 = V stream (transposed into rows), 1 = G stream, 2 = bank U, 3 = zeros
  int64_t n;                      // n_in (V) or n_out (G, U) of the linear
  int32_t r;                      // rank
  int32_t col0;                   // first destination column (G/U: column offset in a Bs row)
  int32_t row_map;                // 0 plain, 1 = gate rows of a 16-interleaved pack, 2 = up rows
  int32_t dtype;                  // 0 f32, 1 bf16, 2 bf16 of v * 2^11 (factor columns of fp8 models)
  int64_t split;                  // bf16 only: 0, or write hi | hi | lo copies `split` elements apart
};
hipError_t launch_side_jobs(const SideJob* jobs_dev, int n_jobs, int64_t max_items, hipStream_t s);

constexpr int ZO_MAX_UPDATE_DIRS = 16;
struct UpdateArgs {                // U <- fp32(U - coef_d * G_d) for every (layer, kind, direction)
  float* u_base;                   // bank memory
  int64_t layer_stride;            // floats per layer within one slot
  int32_t n_kinds;
  int32_t kind_id[7];
  int64_t kind_off[7];             // float offset of the kind within a layer
  int64_t kind_n[7];               // n_out * r
  int32_t n_dirs;
  uint64_t t;                      // step (G stream tau)
  uint64_t seed[ZO_MAX_UPDATE_DIRS];
  int64_t slot_off[ZO_MAX_UPDATE_DIRS];
  double coef[ZO_MAX_UPDATE_DIRS]; // (lr / q) * c_d
  int32_t fresh[ZO_MAX_UPDATE_DIRS];
};
hipError_t launch_update(const UpdateArgs& a, int n_layers, int64_t max_n, hipStream_t s);
hipError_t launch_stream_rowmajor(const SideJob& jb, hipStream_t s);   // stream (seed, tag, tau) -> fp32 [n x r]

struct FoldArgs {                  // W <- round(W + U V^T) of one target linear
  void* w;                         // weight rows (physical layout)
  int64_t ld;                      // physical row pitch (elements)
  int64_t n_out, n_in;
  int32_t layout;                  // 0 plain, 1 gate / 2 up of a 16-row interleave
  int32_t dtype;                   // weight storage: 0 fp32, 1 bf16, 2 e4m3 codes of w * 2^11
  int32_t r;
  const float* u;                  // [n_out x r]
  const float* v;                  // [n_in x r]
};
hipError_t launch_fold(const FoldArgs& a, hipStream_t s);

// ---- transformer pieces ------------------------------------------------------
// token ids outside [0, vocab) are clamped and set *bad (when bad is not null)
template <typename TW>
hipError_t launch_embed_t(const TW* E, const TW* P, const int32_t* tokens, const int32_t* row_src,
                          const int32_t* row_pos, int M, int d, int vocab, float* h, int32_t* bad, hipStream_t s);
template <typename T>
hipError_t launch_norm(const float* h, const int32_t* rows, int M, int d, const float* w, const float* b,
                       float eps, bool rms, T* out, int64_t ld_out, int lo_off, hipStream_t s);
// norm (as launch_norm, no row list, no two-term output) fused with the side input t of the
// projections reading its output: p carries the V^T rows (B, ldb) and the tproj_out fields;
// n_used (1..16) used columns of tp_used per block of tp_ks
template <typename T>
hipError_t launch_norm_side(const float* h, int M, int d, const float* w, const float* b, float eps, bool rms, T* out,
                            int64_t ld_out, const GemmParams& p, int n_used, hipStream_t s);
template <typename T>
hipError_t launch_qknorm_rope(T* qkv, int M, int ld, int hq, int hkv, int hd, const float* qw, const float* kw,
                              float eps, const float2* rope_cs, const int32_t* row_pos, hipStream_t s);
template <typename T>
hipError_t launch_attention(const T* qkv, int ld_qkv, T* out, int ld_out, const int32_t* cu_seqlens, int n_seq,
                            const int32_t* work, int n_work, int hq, int hkv, int hd, hipStream_t s);
template <>
hipError_t launch_attention<bf16_t>(const bf16_t* qkv, int ld_qkv, bf16_t* out, int ld_out, const int32_t* cu,
                                    int n_seq, const int32_t* work, int n_work, int hq, int hkv, int hd,
                                    hipStream_t s);
template <>
hipError_t launch_attention<float>(const float* qkv, int ld_qkv, float* out, int ld_out, const int32_t* cu,
                                   int n_seq, const int32_t* work, int n_work, int hq, int hkv, int hd,
                                   hipStream_t s);
// fp32 q|k|v -> attention output as the two-term bf16 expansion (hi at column c, lo at c + lo_off)
// bf16 q|k|v, output as e4m3 codes (fp8 models)
hipError_t launch_attention_e4m3(const bf16_t* qkv, int ld_qkv, e4m3_t* out, int ld_out, const int32_t* cu,
                                 const int32_t* work, int n_work, int hq, int hkv, int hd, hipStream_t s);
// ---- generation (decode.hip) --------------------------------------------------
template <typename T>
hipError_t launch_kv_append(const T* qkv, int ld, int M, const int32_t* row_cache, int nq, int nkv, T* kc, T* vc,
                            hipStream_t s);
template <typename T, typename TO>
hipError_t launch_decode_attention(const T* qkv, int ld, const T* kc, const T* vc, const int32_t* kv_first,
                                   const int32_t* row_pos, int M, int hq, int hkv, int hd, TO* out, int ld_out,
                                   int max_keys, hipStream_t s);
hipError_t launch_greedy_reduce(const float2* part, const int32_t* part_idx, int n_tiles, int n_rows,
                                int32_t* next_tok, int32_t* tokens_out, float* logp_out, int n_new, int step,
                                hipStream_t s);
hipError_t launch_attention_split(const float* qkv, int ld_qkv, bf16_t* out, int ld_out, int lo_off,
                                  const int32_t* cu, const int32_t* work, int n_work, int hq, int hkv, int hd,
                                  hipStream_t s);
hipError_t launch_tproj_reduce(const GemmParams& p, hipStream_t s);
// t from the partial sums of an epilogue (sf_part, sf_groups, sf_n) in a fixed order, then the
// side-input store of tproj_out (p carries the tproj fields of the consuming projection)
hipError_t launch_side_part_reduce(const GemmParams& p, hipStream_t s);
hipError_t launch_gather_labels(const int32_t* src, const int32_t* idx, int n, int vocab, int32_t* dst,
                                int32_t* bad, hipStream_t s);
hipError_t launch_logp_reduce(const float2* part, int n_tiles, const float* lab_logit, int n_scored,
                              const int32_t* seq_first, int n_phys, double* tok_logp64, float* tok_logp32,
                              double* seq_logp, hipStream_t s);
