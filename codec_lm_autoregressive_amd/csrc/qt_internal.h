// Internal interface between the C-ABI layer (qt_api.hip) and the gfx950
// kernels (qt_kernels.hip). Not installed; the public ABI is include/qt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace qt {

enum DType { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };   // DT_F16: KV cache only
enum Epi { EPI_STORE = 0, EPI_RESIDUAL = 1, EPI_SWIGLU = 2 };

// Device status word bits (read at the once-per-frame sync).
enum StatusBits : int { ST_NONFINITE = 1, ST_RANGE = 2 };

// Y[m, :] (op)= W · norm(X[m, :]) for m < M.  W is [N, K] row-major
// (nn.Linear layout), f32 or bf16; X, Y fp32.  With EPI_SWIGLU the rows of W
// come in (gate j, up j) pairs and Y[m, j] = silu(gate) * up.
struct LinearArgs {
  const void* W; int wdtype; int N; int K;
  const float* X; long ldx; int M;
  const float* gain; float eps;        // RMSNorm prologue when gain != nullptr
  float* Y; long ldy; int epi;
  float* norm_out; long ld_norm;       // optional copy of the normalised X
  float* row_den;                      // [M] scratch for the matrix-core path (nullptr: not used)
  float* part; long part_floats;       // split-K partial sums for 17..128 rows (nullptr: not used)
  int defer;                           // split K: leave the partial sums for the consumer (no reduce)
  void* xs; long xs_floats;            // > 128 rows: scratch for the bf16 hi/lo split of the
                                       // (normalised) activations, M * K floats (nullptr: not used)
  // Causal convolution as one GEMM (conv_taps > 0; bf16 weights, no gain):
  // K = conv_taps * conv_cin and activation element (t, j * conv_cin + c) is
  // X[(t - (conv_taps - 1 - j) * conv_dil) * ldx + c], the rows before X being
  // readable (zeroed padding); conv_cin a multiple of 32.
  int conv_taps; int conv_cin; int conv_dil;
  // SnakeBeta epilogue (convolutions only): with y the output value (after the
  // residual add), writes y + sin(snake_alpha[col] y)^2 / snake_bden[col]
  // to Y, or y to Y and that value to Y2 (row stride ldy2) when Y2 is set.
  const float* snake_alpha; const float* snake_bden; float* Y2; long ldy2;
};
hipError_t launch_linear(const LinearArgs& a, hipStream_t s);
// K ranges the launch of a would split into (partial sums in a.part: range z,
// row m, column n at part[(z * M + m) * N + n]; with a gain the row sums of
// squares follow at part[Z * M * N + z * M + m]); 1 when it writes Y directly.
int linear_split_ranges(const LinearArgs& a);

// One contiguous run of tokens of one batch row: row, first token (row of the
// activation arrays), token count, first position (before pos_base / row_pos).
struct Run { int row, tok0, ntok, pos0; };

// Per-head QK-RMSNorm + rope of q and k, K/V write into the cache, then causal
// GQA attention of every token of the run over cached positions <= its own.
enum AttnMode { ATT_WRITE_ATTEND = 0, ATT_WRITE = 1, ATT_ATTEND = 2 };
// Greedy selection folded into the code predictor's fused attention +
// o-projection at batch 1: the argmax (lowest id on ties) of `logits` (V <=
// 2048 floats) picks the step's code; the first block commits it (used /
// own at column col), adds row tab_off + code of `tab` ([rows, tab_dim],
// weight dtype) to the feedback row fb, and sets ST_NONFINITE in status on a
// NaN or +inf logit (code 0 then), as the selection kernel does.
struct SelFold {
  const float* logits; int V;
  const void* tab; long tab_off; int tab_dim;
  int* used; int* own; int col;
  float* fb;
  int* status;
};

struct AttnArgs {
  int mode;
  int single_token;                    // run i is token i of row i, at position pos_base + row_pos[i]
  int tok_stride, tok_off;             // single_token with tok_stride > 0: row i's token is activation
                                       // row i * tok_stride + tok_off (q/k/v in, attention out)
  int ntok;                            // single_token: new tokens per row (1, or 2 with tok_stride 2 and
                                       // tok_off 0: activation rows 2 i, 2 i + 1 at pos_base, pos_base + 1)
  const float* rope_rows;              // [rows][d]: cos | sin at each row's position, or nullptr
  const float* qkv; long ld_qkv;       // [T, (nq + 2 nkv) d]
  float* out; long ld_out;             // [T, nq d]
  const float* q_gain; const float* k_gain; float eps; float scale;
  const float* cos; const float* sin;  // [max_pos, d/2]
  void* kc; void* vc; int kvdtype;     // this layer: [rows][nkv][max_pos][d]
  long row_stride; int max_pos;
  const Run* runs; int n_runs; const int* row_pos; int pos_base;
  int nq, nkv, d;
  // single-token decode: q/k/v as split-K partial sums of the RMSNorm'd
  // projection instead of qkv (part_z > 0): value = (sum over z of
  // part[(z * part_rows + row) * ld_qkv + col]) / rms(row), the rms from the
  // partial row sums of squares of part_k inputs and part_eps
  const float* part; int part_z; int part_rows; int part_k; float part_eps;
  // single-token decode over kv_split > 1 key ranges (one block each; the
  // range that holds the new key writes it to the cache): each block leaves
  // its running max, softmax sum and unnormalised output in
  // split_buf[row][kv head][range][head of the group][d + 2], and a second
  // launch combines the ranges in order
  int kv_split; float* split_buf;
  // prefill attend pass (ATT_ATTEND) over runs of at most max_ntok tokens
  // (1 .. kAttnTileTokens) on the matrix cores; 0: the per-token kernel
  int max_ntok;
  // code predictor steps 1..14 at batch 1 (fused attention + o-projection
  // only): the first layer's q/k/v are row `code` of lut (row stride lut_ld,
  // the q/k/v layout) and the residual row is row `code` of xlut (fp32) or,
  // without xlut, of sel.tab; the code comes from the folded selection sel
  const float* lut; long lut_ld; const float* xlut;
  SelFold sel;
  // code predictor steps at batch rows > 1 (attention_reads_lut): row r's
  // q/k/v are row lut_codes[r * lut_code_ld] (clamped to 0 .. lut_rows - 1)
  // of lut instead of the projection's output
  const int* lut_codes; int lut_code_ld; int lut_rows;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// Whether the prefill attend pass has the tiled matrix-core kernel for this
// head shape and cache type (runs of up to kAttnTileTokens tokens).
constexpr int kAttnTileTokens = 32;
bool attn_prefill_tiles(int d, int nq, int nkv, int kvdtype);
// Single-token code-predictor attention (one batch row, <= 16 positions)
// fused with the o-projection o (x += W_o . attention, o.X == a.out, bf16
// weights, 16-bit cache). Returns hipErrorNotSupported, doing nothing, for
// other shapes.
hipError_t launch_attention_oproj(const AttnArgs& a, const LinearArgs& o, hipStream_t s);
// Whether launch_attention_oproj takes a folded selection (a.sel) for a code
// predictor of these dimensions: nq 16, nkv 8, head_dim 128, 16-bit cache,
// bf16 weights, V <= 2048 and a multiple of 4, tab_dim <= 2048.
bool attention_oproj_sel_ok(int nq, int nkv, int d, int kvdtype, int wdtype, int V, int tab_dim);
// Whether launch_attention serves a (single-token decode) with the kernel
// that reads q/k/v rows from a code-indexed table (AttnArgs::lut_codes).
bool attention_reads_lut(const AttnArgs& a);

// Per-request settings kept in device memory, so that one captured frame
// graph serves every request of the same batch size.
struct SampParams { int do_sample; float temperature; int top_k; float top_p; float penalty; int min_new; };
struct ReqParams {
  SampParams samp[2];                  // [0] talker, [1] code predictor
  const float* pad;                    // tts_pad row (device)
};

// Logits processing + selection for one batch of rows (one block per row).
// With req != nullptr the sampling settings, seed, max_frames and text / pad
// pointers are read from req (samp[which]) instead of the fields below.
struct SelectArgs {
  const ReqParams* req; int which;
  const float* logits; long ld; int V; int B;
  int row0;                            // the launch covers rows row0 .. row0 + B - 1
  // talker processors
  int processors;
  uint32_t* seen; int seen_words;
  float penalty; int min_new; int eos; int sup_b; int sup_e;
  // warpers
  int do_sample; float temperature; int top_k; float top_p;
  // noise: key (seed, 0), counter (id, stream, selection index, noise row);
  // per-row seeds / noise rows when row_seed / noise_row are given, else
  // `seed` and the row itself; selection index = ctr[row] + ctr_add
  uint64_t seed; int stream; const int* ctr; int ctr_add;
  const uint64_t* row_seed; const int* noise_row;
  // debug inputs (nullable): explicit Exp(1) noise / probabilities [B, V]
  const float* noise_in; const float* probs_in;
  // outputs
  const int* forced; int forced_ld; int forced_col;   // teacher forcing (nullable)
  int* used; int used_ld; int used_col;                // code that feeds the model
  int* own; int own_ld; int own_col;                   // the kernel's own choice (nullable)
  float* processed_out;                                 // debug: processed logits [B, V]
  int* status;
  // epilogue 1: code predictor (next input row, feedback sum)
  int epi;
  const void* tab; int tab_dtype; int tab_dim; long tab_off;
  float* next_in; long next_ld;
  float* fb; long fb_ld;
  // trailing text: row r adds text_ptr[r][frame_k[r]] while frame_k[r] < text_len[r], then the pad row
  int add_text; const float* const* text_ptr; const int* text_len; const float* pad;
  const int* frame_k;                  // per-row frame counters
  // epilogue 2: talker lookahead, finish state (length once frame_k[r] + 1
  // reaches row_max[r], or max_frames without per-row caps)
  int* finished; int* state; int max_frames; const int* row_max;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

// Frame start: commit code 0 per row (forced / EOS for finished rows), mark
// it seen, start the feedback sum, build the 2-token predictor pass-0 input.
struct FrameStartArgs {
  int B; int eos; int V;
  const int* code0_next; const int* finished; const int* forced; int forced_ld;
  uint32_t* seen; int seen_words;
  int* codes;                          // [B, 16]
  const void* temb; int tdtype; int H; // talker codec table [V, H]
  const float* h;                      // [B, H] talker hidden for pass 0
  float* pass0; long pass0_ld;         // [2B, H]
  float* fb; long fb_ld;               // [B, H]
  int* status;
  // cos | sin rows of the talker's position this frame, for its attention
  const float* cos; const float* sin; const int* pos; int half; float* rope_rows;
};
hipError_t launch_frame_start(const FrameStartArgs& a, hipStream_t s);

// Frame end: per-row frame counters and talker positions advance by one
// (rows that have finished stay where they ended).
hipError_t launch_frame_advance(int* frame_k, int* pos, const int* finished, int B, hipStream_t s);

// Row gather / scatter copies dst[i] = src[idx[i]] (fp32 rows of width n).
// Rows of code-indexed tables: for each of the B rows, code = codes[r *
// code_ld] (clamped to 0 .. C - 1), qkv row r = lut row code (n floats) and,
// with xlut, x row r = xlut row code (nx floats).
hipError_t launch_lut_rows(const int* codes, int code_ld, int B, int C, const float* lut, int n, float* qkv,
                           long ld_qkv, const float* xlut, int nx, float* x, long ldx, hipStream_t s);
hipError_t launch_copy_rows(const float* src, long ld_src, const int* idx, int count,
                            float* dst, long ld_dst, int n, hipStream_t s);

// Copy/convert [rows, n] from f32 or bf16 into the packed weight layout.
hipError_t launch_convert(const void* src, int sdtype, long ld_src, void* dst, int ddtype, long ld_dst,
                          long rows, int n, hipStream_t s);
// Exp(1) noise of the selection kernel for n counters (mode 0: [n][4] words
// (vocab id, stream, selection index, row), key (seed, 0)) or n raw 64-bit
// words (mode 1).
hipError_t launch_noise(const uint64_t* in, int mode, uint64_t seed, float* out, long n, hipStream_t s);
// Token-id frontend: X[i] = float(embed[ids[i]]) (zeros for ids[i] < 0),
// rows of `width` (a multiple of 8) elements of type wdtype.
hipError_t launch_gather_rows(const void* embed, int wdtype, int width, const int* ids, int n, float* X, hipStream_t s);
// Hd[i] = silu(Hd[i] + b) over n rows of `width` (a multiple of 4); b may be null.
hipError_t launch_bias_silu(float* Hd, int n, int width, const float* b, hipStream_t s);
// out[i] = (tids[i] >= 0 ? Y[i] + b2 : 0) + (cids[i] >= 0 ? codec[cids[i]] : 0) + (extra ? extra[i] : 0),
// n rows of `width` (a multiple of 4) floats; codec rows of type wdtype; b2 and extra may be null.
hipError_t launch_assemble_rows(const float* Y, const float* b2, const int* tids, const int* cids, const void* codec,
                                int wdtype, const float* extra, float* out, int n, int width, hipStream_t s);
// Fill an int32 buffer.
hipError_t launch_fill_i32(int* p, int v, long n, hipStream_t s);

}  // namespace qt
