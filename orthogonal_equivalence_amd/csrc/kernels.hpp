// Launchers of the non-GEMM kernels (aux.hip). All launch on `stream` and
// return false only for an argument combination they do not handle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// out[ro][i] = in[ri][cidx[i]] for i < ncols, rows r < nrows, with
// ri = rmap_in ? rmap_in[r] : r and ro = rmap_out ? rmap_out[r] : r.
// esize = element bytes (1, 2 or 4); ncols % 8 == 0. Indices are clamped to
// [0, ncols) and [0, nrows).
bool gather_cols(const void* in, int64_t ld_in, const int32_t* rmap_in, void* out, int64_t ld_out,
                 const int32_t* rmap_out, const int32_t* cidx, int64_t ncols, int64_t nrows, int esize,
                 hipStream_t stream);

// inv[perm[i]] = i (perm entries clamped to [0, n)).
void inverse_perm(const int32_t* perm, int32_t* inv, int64_t n, hipStream_t stream);

// out[i] = in[idx[i]] (float), idx clamped to [0, n).
void gather_f32(const float* in, const int32_t* idx, float* out, int64_t n, hipStream_t stream);

// out (cols x rows) = transpose of in (rows x cols), element bytes 1, 2 or 4.
bool transpose(const void* in, void* out, int64_t rows, int64_t cols, int esize, hipStream_t stream);

// Zero n floats (a fill kernel, safe inside captured graphs).
void fill_zero_f32(float* p, int64_t n, hipStream_t stream);

// Skew blocks from packed parameters: Qf[z] (b x b, float) and, if Qh is not
// null, a bfloat16 copy. Block z has size r = min(b, dim - z*b) and packed
// offset z*b(b-1)/2; entries outside r x r are zero.
void unpack_skew(const float* q, int64_t dim, int b, int nblk, float* Qf, uint16_t* Qh, hipStream_t stream);

// S = 2 Q + Q2, written as bfloat16 (Sh) or float (Sf), n elements.
void cnp_mid(const float* Qf, const float* Q2f, uint16_t* Sh, float* Sf, int64_t n, hipStream_t stream);

// G - I = 2Q + 2Q2 + T per block, written as plane 0 (row-major) and plane 1
// (transposed) of the CNP block buffer in bfloat16 (bf16 = true) or float.
void cnp_finish(const float* Qf, const float* Q2f, const float* Tf, int b, int nblk, void* gbuf, bool bf16,
                hipStream_t stream);

// dQ = 2U - 2W1 + 2W2 - W3 and dq[k(i,l)] = dQ[i][l] - dQ[l][i] (i < l < r).
void cnp_bwd_pack(const float* U, const float* W1, const float* W2, const float* W3, int64_t dim, int b,
                  int nblk, float* dq, hipStream_t stream);

// out[e] = sum_{s < nsplit} part[s * n + e] (fixed order); optional bf16 copy.
void reduce_splits(const float* part, int nsplit, int64_t n, float* out, uint16_t* out_h, hipStream_t stream);

}  // namespace poetx
