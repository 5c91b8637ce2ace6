#include "device.hpp"
namespace ets {
bool sparse_supported(int H, int dqk, int dv) { (void)H; (void)dqk; (void)dv; return false; }
int launch_sparse_fwd(const SparseArgs&, Dt, void*) { return (int)hipErrorNotSupported; }
int launch_sparse_bwd(const SparseArgs&, Dt, void*) { return (int)hipErrorNotSupported; }
}  // namespace ets
