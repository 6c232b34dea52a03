// Internal declarations shared by the host-side translation units of libsvdq.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <vector>

namespace svdq {

// Thread-local "last error" message behind svdq_last_error().
void set_error(const char* fmt, ...);
void clear_error();

// Symmetric eigen-solver on a dense n x n matrix (row-major, overwritten).
// Computes the `r` largest eigenvalues (descending) and their eigenvectors
// (Z: n x r, row-major, column j belongs to eval[j]). When all_evals is not
// null it also receives all n eigenvalues, descending. Returns false if the
// inverse iteration does not converge.
bool sym_top_eigen(std::vector<double>& A, int64_t n, int r, std::vector<double>& eval,
                   std::vector<double>& Z, std::vector<double>* all_evals);

// A KH x KW convolution over an NHWC image, seen as the linear layer on its
// patch matrix (M = batch*OH*OW rows, K = KH*KW*C columns).
struct ConvShape {
  int64_t batch, H, W, C;
  int32_t KH, KW, stride, pad;
  int64_t OH, OW, M, K;
};

// Checks a convolution's sizes and fills `cs`: C a positive multiple of 64,
// KH, KW, stride in [1, 64], pad in [0, 64], at least one output pixel, and
// image and patch matrix indexable with 32-bit element offsets. Returns a
// status (SVDQ_OK or SVDQ_ERR_SHAPE) and sets the error message.
int check_conv(int64_t batch, int64_t H, int64_t W, int64_t C, int32_t KH, int32_t KW,
               int32_t stride, int32_t pad, ConvShape& cs, const char* fn);

// G = B . B^T for B: n x m row-major (G: n x n, full storage).
void gram_rows(const double* B, int64_t n, int64_t m, double* G);

}  // namespace svdq
