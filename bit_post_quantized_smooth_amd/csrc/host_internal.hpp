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

// G = B . B^T for B: n x m row-major (G: n x n, full storage).
void gram_rows(const double* B, int64_t n, int64_t m, double* G);

}  // namespace svdq
