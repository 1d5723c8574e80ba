// ham_rnn_chunked.hip -- placeholder until the chunked kernel lands.
#include "ham_common.h"
#include "ham_internal.h"
namespace ham {
bool rnn_chunked_supported(int, int, int) { return false; }
int rnn_chunked_slices(int dv) { return dv / 16; }
hipError_t launch_rnn_chunked(int, int, int, const RnnArgs&, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace ham
