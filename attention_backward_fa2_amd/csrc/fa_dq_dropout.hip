// fa_dq_dropout.hip -- the dropout instantiations of the dQ kernel of
// fa_dq.hip, in a translation unit of their own so that they compile in
// parallel with the rest.
#define FA_TU_DROPOUT 1
#include "fa_dq.hip"
