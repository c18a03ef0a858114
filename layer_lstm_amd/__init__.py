"""MI355X-native single-layer LSTM forward + backpropagation through time.

The compute path is the C-ABI library ``liblstm.so`` (hand-written HIP for
gfx950) declared in ``include/lstm.h``; ``layer_lstm_amd.lstm`` is its thin
ctypes binding, ``layer_lstm_amd.synth`` the seeded input generator.
Importing the package loads neither.
"""
